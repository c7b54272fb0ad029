// Grouped GEMM with float32 FMA on the vector ALUs (fp32 layer, and the
// router's float32 products x W_r^T, dl^T x and dl W_r). Same grouping,
// tile scheduling and epilogues as the bf16 matrix-core kernel; operands may
// be bf16 or float32 in HBM and are widened to float32 in LDS.
//
// Workgroup: 256 threads in a 16x16 grid, tile BM x BN x 16, each thread an
// (BM/16) x (BN/16) register block. LDS holds both operands k-major
// ([16][BM] and [16][BN]) so the inner loop reads float4 rows.
// Optional split-K (RAG_NONE only): partition s of gridDim.y writes its
// partial tile to C + s*M*ldc, summed afterwards in a fixed order.
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

// Router products (single group, float32 out).
//  logits    = x W_r^T : A = x (dt, K-major), B = W_r (float, K-major)
//  dw_r      = dl^T x  : A = dl (float, K-strided), B = x (dt, K-strided), split-K
//  dx_router = dl W_r  : A = dl (float, K-major), B = W_r (float, K-strided)
hipError_t gemm_router_logits(const GemmArgs& p, bool x_bf16, hipStream_t s) {
  if (x_bf16)
    return launch_f32<bf16_t, float, float, 64, 64, true, true, EPI_STORE, RAG_NONE>(p, s);
  return launch_f32<float, float, float, 64, 64, true, true, EPI_STORE, RAG_NONE>(p, s);
}
hipError_t gemm_router_dw(const GemmArgs& p, bool x_bf16, hipStream_t s) {
  if (x_bf16)
    return launch_f32<float, bf16_t, float, 64, 64, false, false, EPI_STORE, RAG_NONE>(p, s);
  return launch_f32<float, float, float, 64, 64, false, false, EPI_STORE, RAG_NONE>(p, s);
}
hipError_t gemm_router_dx(const GemmArgs& p, hipStream_t s) {
  return launch_f32<float, float, float, 64, 64, true, false, EPI_STORE, RAG_NONE>(p, s);
}

}  // namespace moe
