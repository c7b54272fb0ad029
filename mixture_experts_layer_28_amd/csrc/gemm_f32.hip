// Grouped GEMM with float32 FMA on the vector ALUs (fp32 layer, and the
// router's float32 products x W_r^T, dl^T x and dl W_r). Same grouping,
// tile scheduling and epilogues as the bf16 matrix-core kernel; operands may
// be bf16 or float32 in HBM and are widened to float32 in LDS.
//
// Workgroup: 256 threads in a 16x16 grid, tile BM x BN x 16, each thread an
// (BM/16) x (BN/16) register block. LDS holds both operands k-major
// ([16][BM] and [16][BN]) so the inner loop reads float4 rows.
// Optional split-K (RAG_NONE only): partition s of gridDim.y writes its
// partial tile to C + s*M*ldc, summed afterwards in a fixed order; a column
// bias goes into partition 0 only.
#include "gemm_tile.h"

namespace moe {

constexpr int kFK = 16;

template <typename TA, typename TB, typename TC, int BM, int BN, bool AKM, bool BKM, int EPI,
          int RAG>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs p) {
  constexpr int TM = BM / 16, TN = BN / 16;
  constexpr bool FUSED = EPI == EPI_SWIGLU_FWD;
  constexpr int BNo = FUSED ? BN / 2 : BN;
  constexpr int PA = BM + 4, PB = BN + 4;           // LDS row strides
  constexpr int TILE_FL = 2 * kFK * (PA + PB);
  constexpr int LDST = BN + 4;
  constexpr int STAGE_FL = BM * LDST;
  constexpr int SMEM_FL = TILE_FL > STAGE_FL ? TILE_FL : STAGE_FL;
  __shared__ __attribute__((aligned(16))) float smem[SMEM_FL];
  __shared__ int s_tiles[1028];
  __shared__ int s_wsum[4];

  Tile t;
  if (!resolve_tile<BM, BNo, RAG>(p, s_tiles, s_wsum, t)) return;

  int64_t kbeg = 0, kend = t.K;
  TC* c_save = reinterpret_cast<TC*>(p.c);
  GemmArgs q = p;
  if (RAG == RAG_NONE && p.k_splits > 1) {
    const int64_t per = ((t.K + p.k_splits - 1) / p.k_splits + kFK - 1) / kFK * kFK;
    kbeg = blockIdx.y * per;
    kend = kbeg + per < t.K ? kbeg + per : t.K;
    q.c = c_save + (int64_t)blockIdx.y * p.G * p.M * p.ldc;
    if (blockIdx.y != 0) q.col_bias = nullptr;   // the bias goes into partition 0 only
  }

  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const TA* Ab = operand_base<TA>(p.a, t);
  const TB* Bb = operand_base<TB>(p.b, t);
  constexpr int FBUF = kFK * (PA + PB);   // buffer b: A at smem + b*FBUF, B after it

  float acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;

  constexpr int NA = BM * kFK / 256, NB = BN * kFK / 256;
  float ra[NA], rb[NB];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int e = tid + 256 * i;
      int m, kk;
      if (AKM) { m = e / kFK; kk = e % kFK; } else { kk = e / BM; m = e % BM; }
      const int64_t gm = t.m0 + m, gk = k0 + kk;
      const bool ok = gm < t.M && gk < kend;
      ra[i] = ok ? to_f(AKM ? Ab[gm * p.a.ld + gk] : Ab[gk * p.a.ld + gm]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int e = tid + 256 * i;
      int n, kk;
      if (BKM) { n = e / kFK; kk = e % kFK; } else { kk = e / BN; n = e % BN; }
      int64_t gn;
      bool ok;
      if (FUSED) {
        const int half = BN / 2;
        const int64_t col = t.n0 + (n < half ? n : n - half);
        ok = col < p.fdim;
        gn = n < half ? col : p.fdim + col;
      } else {
        gn = t.n0 + n;
        ok = gn < p.N;
      }
      const int64_t gk = k0 + kk;
      ok = ok && gk < kend;
      rb[i] = ok ? to_f(BKM ? Bb[gn * p.b.ld + gk] : Bb[gk * p.b.ld + gn]) : 0.f;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int e = tid + 256 * i;
      int m, kk;
      if (AKM) { m = e / kFK; kk = e % kFK; } else { kk = e / BM; m = e % BM; }
      smem[buf * FBUF + kk * PA + m] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int e = tid + 256 * i;
      int n, kk;
      if (BKM) { n = e / kFK; kk = e % kFK; } else { kk = e / BN; n = e % BN; }
      smem[buf * FBUF + kFK * PA + kk * PB + n] = rb[i];
    }
  };

  const int64_t nk = kend > kbeg ? (kend - kbeg + kFK - 1) / kFK : 0;
  if (nk > 0) {
    load(kbeg);
    store(0);
    __syncthreads();
  }
  for (int64_t it = 0; it < nk; ++it) {
    const int cur = it & 1;
    if (it + 1 < nk) load(kbeg + (it + 1) * kFK);
    const float* as = smem + cur * FBUF;
    const float* bs = as + kFK * PA;
#pragma unroll
    for (int kk = 0; kk < kFK; ++kk) {
      float av[TM], bv[TN];
#pragma unroll
      for (int i = 0; i < TM; i += 4) {
        float4 v = *reinterpret_cast<const float4*>(as + kk * PA + ty * TM + i);
        av[i] = v.x; av[i + 1] = v.y; av[i + 2] = v.z; av[i + 3] = v.w;
      }
#pragma unroll
      for (int j = 0; j < TN; j += 4) {
        float4 v = *reinterpret_cast<const float4*>(bs + kk * PB + tx * TN + j);
        bv[j] = v.x; bv[j + 1] = v.y; bv[j + 2] = v.z; bv[j + 3] = v.w;
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    if (it + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  // stage the whole tile, then the row-contiguous epilogue with 256 threads
  float* stage = smem;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; j += 4)
      *reinterpret_cast<float4*>(stage + (ty * TM + i) * LDST + tx * TN + j) =
          make_float4(acc[i][j], acc[i][j + 1], acc[i][j + 2], acc[i][j + 3]);
  __syncthreads();
  if (FUSED)
    epilogue_rows<TC, EPI>(q, t, stage, LDST, BM, BN / 2, t.m0, t.n0, tid, 256);
  else
    epilogue_rows<TC, EPI>(q, t, stage, LDST, BM, BN, t.m0, t.n0, tid, 256);
}

template <typename TA, typename TB, typename TC, int BM, int BN, bool AKM, bool BKM, int EPI,
          int RAG>
static hipError_t launch_f32(const GemmArgs& p, hipStream_t s) {
  constexpr int BNo = EPI == EPI_SWIGLU_FWD ? BN / 2 : BN;
  const int64_t nt = (p.N + BNo - 1) / BNo;
  int64_t tiles;
  if (RAG == RAG_M)
    tiles = ((p.max_rows + BM - 1) / BM + p.G) * nt;
  else
    tiles = (int64_t)p.G * ((p.M + BM - 1) / BM) * nt;
  if (tiles == 0) return hipSuccess;
  const int64_t nb = RAG == RAG_K ? rag_k_grid(p.G, ((p.M + BM - 1) / BM) * nt)
                                  : (tiles + 7) / 8 * 8;
  const unsigned ny = (RAG == RAG_NONE && p.k_splits > 1) ? (unsigned)p.k_splits : 1u;
  hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, TC, BM, BN, AKM, BKM, EPI, RAG>),
                     dim3((unsigned)nb, ny), dim3(256), 0, s, p);
  return hipGetLastError();
}

// fp32 layer: all operands float. Tile 64x64 (small problems, ragged rows).
hipError_t gemm_f32(const GemmArgs& p, bool akm, bool bkm, int epi, int rag, hipStream_t s) {
#define MOE_CASE(AK, BK_, E_, R_)                                              \
  if (akm == AK && bkm == BK_ && epi == E_ && rag == R_)                       \
    return launch_f32<float, float, float, 64, 64, AK, BK_, E_, R_>(p, s);
  MOE_CASE(true, true, EPI_SWIGLU_FWD, RAG_M)
  MOE_CASE(true, true, EPI_GELU_FWD, RAG_M)
  MOE_CASE(true, true, EPI_STORE, RAG_M)
  MOE_CASE(true, false, EPI_SWIGLU_BWD, RAG_M)
  MOE_CASE(true, false, EPI_GELU_BWD, RAG_M)
  MOE_CASE(true, false, EPI_STORE, RAG_M)
  MOE_CASE(false, false, EPI_STORE, RAG_K)
  MOE_CASE(true, true, EPI_SWIGLU_FWD, RAG_NONE)
  MOE_CASE(true, true, EPI_GELU_FWD, RAG_NONE)
  MOE_CASE(true, true, EPI_STORE, RAG_NONE)
  MOE_CASE(true, false, EPI_SWIGLU_BWD, RAG_NONE)
  MOE_CASE(true, false, EPI_GELU_BWD, RAG_NONE)
  MOE_CASE(true, false, EPI_STORE, RAG_NONE)
  MOE_CASE(false, false, EPI_STORE, RAG_NONE)
#undef MOE_CASE
  return hipErrorInvalidValue;
}

// ---------------------------------------------- router products on MFMA
// float32 matrix-core variant of the kernel above for the router's products
// (single group, plain store, optional split-K): v_mfma_f32_32x32x2_f32 at
// twice the vector ALU's float32 rate, full float32 operands and accumulation.
// Tile 64 x 64 x 32; wave w owns the 32 x 32 quarter (w & 1, w >> 1). LDS
// holds both operands k-major with a row stride of 96 floats, so the two
// k rows one MFMA reads (lanes 0-31 and 32-63) fall in disjoint banks.
// Global loads take 8 consecutive elements per thread (one 16-byte load for
// bf16, two for float32), which needs 16-byte aligned bases and leading
// dimensions that are multiples of 8 (checked by the dispatcher); partial
// vectors at the K or row edge fall back to element loads.
constexpr int kMK = 32, kMP = 96;

// Eight consecutive elements of T kept as raw words between a slab's global
// load and its LDS store (converting at load time would make the load's
// branch wait for the data).
template <typename T> struct Raw8 { uint32_t w[sizeof(T) * 2]; };
__device__ __forceinline__ float raw8_get(const Raw8<bf16_t>& r, int i) {
  return bf2f((i & 1) ? r.w[i >> 1] >> 16 : r.w[i >> 1] & 0xffff);
}
__device__ __forceinline__ float raw8_get(const Raw8<float>& r, int i) {
  return __uint_as_float(r.w[i]);
}

// Slab loader for one operand. KM: rows are k-contiguous (X[row][k]); else
// row-contiguous (X[k][row]). Thread layout keeps each wave's LDS stores on
// distinct banks: KM takes row = tid & 63 and k-octet tid >> 6; row-contiguous
// takes k = tid >> 3 and row-octet tid & 7. Elements past the K or row edge
// read as zero.
template <typename T, bool KM>
__device__ __forceinline__ void mfma_slab_load(const T* base, int64_t ld, int64_t r0, int64_t rows,
                                               int64_t k0, int64_t kend, int tid, Raw8<T>& v) {
  int64_t row, k;
  int nv;
  if (KM) {
    row = r0 + (tid & 63);
    k = k0 + (tid >> 6) * 8;
    const int64_t rem = kend - k;
    nv = row < rows ? (rem >= 8 ? 8 : (rem > 0 ? (int)rem : 0)) : 0;
  } else {
    k = k0 + (tid >> 3);
    row = r0 + (tid & 7) * 8;
    const int64_t rem = rows - row;
    nv = k < kend ? (rem >= 8 ? 8 : (rem > 0 ? (int)rem : 0)) : 0;
  }
  const T* src = base + (KM ? row * ld + k : k * ld + row);
  constexpr int NW = sizeof(T) * 2;
  if (nv == 8) {
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const uint4 u = s4[i];
      v.w[4 * i] = u.x; v.w[4 * i + 1] = u.y; v.w[4 * i + 2] = u.z; v.w[4 * i + 3] = u.w;
    }
  } else {
    const uint32_t* s32 = reinterpret_cast<const uint32_t*>(src);
    const uint16_t* s16 = reinterpret_cast<const uint16_t*>(src);
#pragma unroll
    for (int i = 0; i < NW; ++i) v.w[i] = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < nv) {
        if (sizeof(T) == 4) v.w[i] = s32[i];
        else v.w[i >> 1] |= (uint32_t)s16[i] << (16 * (i & 1));
      }
    }
  }
}

template <typename T, bool KM>
__device__ __forceinline__ void mfma_slab_store(float* s, int tid, const Raw8<T>& v) {
  if (KM) {
    const int r = tid & 63, kq = (tid >> 6) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) s[(kq + j) * kMP + r] = raw8_get(v, j);
  } else {
    float* d = s + (tid >> 3) * kMP + (tid & 7) * 8;
    reinterpret_cast<float4*>(d)[0] =
        make_float4(raw8_get(v, 0), raw8_get(v, 1), raw8_get(v, 2), raw8_get(v, 3));
    reinterpret_cast<float4*>(d)[1] =
        make_float4(raw8_get(v, 4), raw8_get(v, 5), raw8_get(v, 6), raw8_get(v, 7));
  }
}

template <typename TA, typename TB, bool AKM, bool BKM>
__global__ __launch_bounds__(256) void gemm_f32_mfma_kernel(GemmArgs p) {
  constexpr int BM = 64, BN = 64, LDST = BN + 4;
  constexpr int FBUF = 2 * kMK * kMP;      // buffer b: A at smem + b*FBUF, B after it
  __shared__ __attribute__((aligned(16))) float smem[2 * FBUF];
  __shared__ int s_tiles[1028];
  __shared__ int s_wsum[4];

  Tile t;
  if (!resolve_tile<BM, BN, RAG_NONE>(p, s_tiles, s_wsum, t)) return;

  int64_t kbeg = 0, kend = t.K;
  GemmArgs q = p;
  if (p.k_splits > 1) {
    const int64_t per = ((t.K + p.k_splits - 1) / p.k_splits + kMK - 1) / kMK * kMK;
    kbeg = blockIdx.y * per;
    kend = kbeg + per < t.K ? kbeg + per : t.K;
    q.c = reinterpret_cast<float*>(p.c) + (int64_t)blockIdx.y * p.G * p.M * p.ldc;
    if (blockIdx.y != 0) q.col_bias = nullptr;   // the bias goes into partition 0 only
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const TA* Ab = operand_base<TA>(p.a, t);
  const TB* Bb = operand_base<TB>(p.b, t);
  // this lane's operand element within a 2-deep k step: row/col lane & 31, k lane >> 5
  const int aoff = (lane >> 5) * kMP + (wave & 1) * 32 + (lane & 31);
  const int boff = kMK * kMP + (lane >> 5) * kMP + (wave >> 1) * 32 + (lane & 31);

  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;

  Raw8<TA> ra;
  Raw8<TB> rb;
  const int64_t nk = kend > kbeg ? (kend - kbeg + kMK - 1) / kMK : 0;
  if (nk > 0) {
    mfma_slab_load<TA, AKM>(Ab, p.a.ld, t.m0, t.M, kbeg, kend, tid, ra);
    mfma_slab_load<TB, BKM>(Bb, p.b.ld, t.n0, p.N, kbeg, kend, tid, rb);
    mfma_slab_store<TA, AKM>(smem, tid, ra);
    mfma_slab_store<TB, BKM>(smem + kMK * kMP, tid, rb);
    __syncthreads();
  }
  for (int64_t it = 0; it < nk; ++it) {
    const int cur = it & 1;
    if (it + 1 < nk) {
      const int64_t k0 = kbeg + (it + 1) * kMK;
      mfma_slab_load<TA, AKM>(Ab, p.a.ld, t.m0, t.M, k0, kend, tid, ra);
      mfma_slab_load<TB, BKM>(Bb, p.b.ld, t.n0, p.N, k0, kend, tid, rb);
    }
    const float* sb = smem + cur * FBUF;
    float av[kMK / 2], bv[kMK / 2];
#pragma unroll
    for (int i = 0; i < kMK / 2; ++i) {
      av[i] = sb[aoff + 2 * i * kMP];
      bv[i] = sb[boff + 2 * i * kMP];
    }
    __builtin_amdgcn_sched_barrier(0);   // all LDS reads in flight before the MFMA chain
#pragma unroll
    for (int i = 0; i < kMK / 2; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i], bv[i], acc, 0, 0, 0);
    if (it + 1 < nk) {
      mfma_slab_store<TA, AKM>(smem + (cur ^ 1) * FBUF, tid, ra);
      mfma_slab_store<TB, BKM>(smem + (cur ^ 1) * FBUF + kMK * kMP, tid, rb);
    }
    __syncthreads();
  }

  // accumulator register r of lane l is C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]
  // of the wave's quarter; stage the tile, then the shared row epilogue
  float* stage = smem;
  const int sr = (wave & 1) * 32 + 4 * (lane >> 5), sc = (wave >> 1) * 32 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) stage[(sr + 8 * (r >> 2) + (r & 3)) * LDST + sc] = acc[r];
  __syncthreads();
  epilogue_rows<float, EPI_STORE>(q, t, stage, LDST, BM, BN, t.m0, t.n0, tid, 256);
}

template <typename TA, typename TB, bool AKM, bool BKM>
static hipError_t launch_f32_mfma(const GemmArgs& p, hipStream_t s) {
  const int64_t tiles = (int64_t)p.G * ((p.M + 63) / 64) * ((p.N + 63) / 64);
  if (tiles == 0) return hipSuccess;
  const unsigned ny = p.k_splits > 1 ? (unsigned)p.k_splits : 1u;
  hipLaunchKernelGGL((gemm_f32_mfma_kernel<TA, TB, AKM, BKM>), dim3((unsigned)((tiles + 7) / 8 * 8), ny),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

// The matrix-core path's vector loads need 16-byte aligned operand bases and
// leading dimensions that are multiples of 8 elements.
static bool mfma_operands_ok(const GemmArgs& p) {
  auto ok = [](const Operand& o) {
    return ((uintptr_t)o.base & 15) == 0 && (o.ld & 7) == 0;
  };
  return ok(p.a) && ok(p.b);
}

// Router products (single group, float32 out).
//  logits    = x W_r^T : A = x (dt, K-major), B = W_r (float, K-major)
//  dw_r      = dl^T x  : A = dl (float, K-strided), B = x (dt, K-strided), split-K
//  dx_router = dl W_r  : A = dl (float, K-major), B = W_r (float, K-strided)
// Matrix cores when the operands allow their vector loads, else the ALU kernel.
hipError_t gemm_router_logits(const GemmArgs& p, bool x_bf16, hipStream_t s) {
  if (mfma_operands_ok(p))
    return x_bf16 ? launch_f32_mfma<bf16_t, float, true, true>(p, s)
                  : launch_f32_mfma<float, float, true, true>(p, s);
  if (x_bf16)
    return launch_f32<bf16_t, float, float, 64, 64, true, true, EPI_STORE, RAG_NONE>(p, s);
  return launch_f32<float, float, float, 64, 64, true, true, EPI_STORE, RAG_NONE>(p, s);
}
hipError_t gemm_router_dw(const GemmArgs& p, bool x_bf16, hipStream_t s) {
  if (mfma_operands_ok(p))
    return x_bf16 ? launch_f32_mfma<float, bf16_t, false, false>(p, s)
                  : launch_f32_mfma<float, float, false, false>(p, s);
  if (x_bf16)
    return launch_f32<float, bf16_t, float, 64, 64, false, false, EPI_STORE, RAG_NONE>(p, s);
  return launch_f32<float, float, float, 64, 64, false, false, EPI_STORE, RAG_NONE>(p, s);
}
hipError_t gemm_router_dx(const GemmArgs& p, hipStream_t s) {
  if (mfma_operands_ok(p)) return launch_f32_mfma<float, float, true, false>(p, s);
  return launch_f32<float, float, float, 64, 64, true, false, EPI_STORE, RAG_NONE>(p, s);
}

}  // namespace moe
