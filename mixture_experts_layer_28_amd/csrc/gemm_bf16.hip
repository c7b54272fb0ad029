// Grouped GEMM on the bf16 matrix cores of gfx950 (v_mfma_f32_32x32x16_bf16),
// float32 accumulation. One launch covers every expert ("grouped GEMM": each
// expert's GEMM on its own contiguous rows, tiled per expert, one kernel).
//
// Workgroup: 256 threads = 4 waves in a 2x2 grid; tile BM x BN x 64; each
// wave owns a (BM/2) x (BN/2) sub-tile of 32x32 MFMA blocks.
// LDS holds both operands K-contiguous ([rows][64] bf16, 16-byte chunks
// XOR-swizzled by row so the MFMA fragment reads are bank-conflict free),
// double-buffered: global loads of k-tile i+1 are in flight while the
// matrix cores work on tile i. An operand stored K-strided in HBM (the
// transposed reads of the backward) is loaded as 8x8 blocks and transposed
// in registers before the LDS store, so the inner loop is the same for
// every layout.
#include "gemm_tile.h"

namespace moe {

constexpr int kBK = 64;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kBK + ((chunk ^ (row & 7)) << 3);
}

// Load the (ROWS x 64) k-tile of one operand into registers.
// KM: operand K-contiguous in HBM. FUSED: B rows interleave gate/up weight
// rows (fused SwiGLU); row j of the tile -> weight row via fused_row().
template <int ROWS, bool KM>
struct TileLoader {
  static constexpr int NREG = KM ? ROWS / 32 : ((ROWS + 255) / 256) * 8;
  uint4 r[NREG];
};

// weight row of fused tile row j; -1 when beyond f
__device__ __forceinline__ int64_t fused_row(int j, int WN, int64_t n0h, int64_t fdim) {
  const int wc = j / WN, w = j - wc * WN, half = WN >> 1;
  const bool up = w >= half;
  const int64_t col = n0h + wc * half + (up ? w - half : w);
  if (col >= fdim) return -1;
  return up ? fdim + col : col;
}

template <int ROWS, bool KM, bool FUSED, int WN>
__device__ __forceinline__ void load_tile(TileLoader<ROWS, KM>& L, const bf16_t* __restrict__ base,
                                          int64_t ld, int64_t rows_valid, int64_t r0, int64_t k0,
                                          int64_t K, int64_t fdim) {
  const int tid = threadIdx.x;
  if (KM) {
#pragma unroll
    for (int i = 0; i < ROWS / 32; ++i) {
      const int q = tid + 256 * i;
      const int row = q >> 3, ch = q & 7;
      const int64_t kk = k0 + ch * 8;
      int64_t grow;
      bool ok;
      if (FUSED) {
        grow = fused_row(row, WN, r0, fdim);
        ok = grow >= 0;
      } else {
        grow = r0 + row;
        ok = grow < rows_valid;
      }
      ok = ok && kk < K;
      L.r[i] = ok ? *reinterpret_cast<const uint4*>(base + grow * ld + kk) : make_uint4(0, 0, 0, 0);
    }
  } else {
    // K-strided: element (row, kk) at base + kk*ld + row; 8x8 blocks
#pragma unroll
    for (int it = 0; it < (ROWS + 255) / 256; ++it) {
      const int q = tid + 256 * it;
      const int kb = q / (ROWS / 8), mb = q - kb * (ROWS / 8);
      const int64_t grow = r0 + mb * 8;
      const bool okq = q < ROWS && grow < rows_valid;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int64_t kk = k0 + kb * 8 + rr;
        L.r[it * 8 + rr] = (okq && kk < K)
                               ? *reinterpret_cast<const uint4*>(base + kk * ld + grow)
                               : make_uint4(0, 0, 0, 0);
      }
    }
  }
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

template <int ROWS, bool KM>
__device__ __forceinline__ void store_tile(const TileLoader<ROWS, KM>& L, bf16_t* lds) {
  const int tid = threadIdx.x;
  if (KM) {
#pragma unroll
    for (int i = 0; i < ROWS / 32; ++i) {
      const int q = tid + 256 * i;
      const int row = q >> 3, ch = q & 7;
      *reinterpret_cast<uint4*>(lds + swz(row, ch)) = L.r[i];
    }
  } else {
#pragma unroll
    for (int it = 0; it < (ROWS + 255) / 256; ++it) {
      const int q = tid + 256 * it;
      if (q >= ROWS) continue;
      const int kb = q / (ROWS / 8), mb = q - kb * (ROWS / 8);
      const uint4* R = &L.r[it * 8];
      // R[rr] holds k = kb*8+rr for rows mb*8 .. mb*8+7 (2 per dword)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int w = i >> 1;
        auto pick = [&](const uint4& v) -> uint32_t {
          return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
        };
        uint4 o;
        if ((i & 1) == 0) {
          o.x = lo_pair(pick(R[0]), pick(R[1]));
          o.y = lo_pair(pick(R[2]), pick(R[3]));
          o.z = lo_pair(pick(R[4]), pick(R[5]));
          o.w = lo_pair(pick(R[6]), pick(R[7]));
        } else {
          o.x = hi_pair(pick(R[0]), pick(R[1]));
          o.y = hi_pair(pick(R[2]), pick(R[3]));
          o.z = hi_pair(pick(R[4]), pick(R[5]));
          o.w = hi_pair(pick(R[6]), pick(R[7]));
        }
        *reinterpret_cast<uint4*>(lds + swz(mb * 8 + i, kb)) = o;
      }
    }
  }
}

template <int BM, int BN, bool AKM, bool BKM, int EPI, int RAG>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2, MI = WM / 32, NI = WN / 32;
  constexpr bool FUSED = EPI == EPI_SWIGLU_FWD;
  constexpr int BNo = FUSED ? BN / 2 : BN;      // output columns per tile
  constexpr int A_EL = BM * kBK, B_EL = BN * kBK;
  constexpr int LDST = WN + 4;                  // staging row stride (floats)
  static_assert(4 * 32 * LDST * 4 <= 2 * (A_EL + B_EL) * 2, "staging does not fit");
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * (A_EL + B_EL)];
  __shared__ int s_tiles[1028];
  __shared__ int s_wsum[4];

  Tile t;
  if (!resolve_tile<BM, BNo, RAG>(p, s_tiles, s_wsum, t)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
  const bf16_t* Ab = operand_base<bf16_t>(p.a, t);
  const bf16_t* Bb = operand_base<bf16_t>(p.b, t);
  const int64_t a_rows = t.M;                 // valid A rows (m)
  const int64_t b_rows = FUSED ? p.fdim : p.N;

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  TileLoader<BM, AKM> la;
  TileLoader<BN, BKM> lb;
  const int64_t nk = (t.K + kBK - 1) / kBK;
  // buffer b: A at lds + b*(A_EL+B_EL), B right after it
  constexpr int BUF = A_EL + B_EL;

  if (nk > 0) {
    load_tile<BM, AKM, false, WN>(la, Ab, p.a.ld, a_rows, t.m0, 0, t.K, p.fdim);
    load_tile<BN, BKM, FUSED, WN>(lb, Bb, p.b.ld, b_rows, t.n0, 0, t.K, p.fdim);
    store_tile<BM, AKM>(la, lds);
    store_tile<BN, BKM>(lb, lds + A_EL);
    __syncthreads();
  }
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_tile<BM, AKM, false, WN>(la, Ab, p.a.ld, a_rows, t.m0, (kt + 1) * kBK, t.K, p.fdim);
      load_tile<BN, BKM, FUSED, WN>(lb, Bb, p.b.ld, b_rows, t.n0, (kt + 1) * kBK, t.K, p.fdim);
    }
    const bf16_t* as = lds + cur * BUF;
    const bf16_t* bs = as + A_EL;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 af[MI], bfr[NI];
      const int ch = kk * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int row = wm0 + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8*>(as + swz(row, ch));
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int row = wn0 + j * 32 + (lane & 31);
        bfr[j] = *reinterpret_cast<const bf16x8*>(bs + swz(row, ch));
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      store_tile<BM, AKM>(la, lds + (cur ^ 1) * BUF);
      store_tile<BN, BKM>(lb, lds + (cur ^ 1) * BUF + A_EL);
    }
    __syncthreads();
  }

  // ---- epilogue: stage 32 rows of the wave's sub-tile at a time in LDS
  float* stage = reinterpret_cast<float*>(lds) + wave * (32 * LDST);
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3);
        stage[row * LDST + j * 32 + (lane & 31)] = acc[i][j][r];
      }
    __syncthreads();
    const int64_t m0 = t.m0 + wm0 + i * 32;
    if (FUSED)
      epilogue_rows<bf16_t, EPI>(p, t, stage, LDST, 32, WN / 2, m0,
                                 t.n0 + (wave & 1) * (WN / 2), lane, 64);
    else
      epilogue_rows<bf16_t, EPI>(p, t, stage, LDST, 32, WN, m0, t.n0 + wn0, lane, 64);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ launch
template <int BM, int BN, bool AKM, bool BKM, int EPI, int RAG>
static hipError_t launch_one(const GemmArgs& p, hipStream_t s) {
  constexpr int BNo = EPI == EPI_SWIGLU_FWD ? BN / 2 : BN;
  const int64_t nt = (p.N + BNo - 1) / BNo;
  int64_t tiles;
  if (RAG == RAG_M)
    tiles = ((p.max_rows + BM - 1) / BM + p.G) * nt;
  else
    tiles = (int64_t)p.G * ((p.M + BM - 1) / BM) * nt;
  const int64_t nb = (tiles + 7) / 8 * 8;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, AKM, BKM, EPI, RAG>), dim3((unsigned)nb),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

// Dispatch over the layouts/epilogues the layer uses.
hipError_t gemm_bf16(const GemmArgs& p, bool akm, bool bkm, int epi, int rag, hipStream_t s) {
#define MOE_CASE(AK, BK_, E_, R_)                                          \
  if (akm == AK && bkm == BK_ && epi == E_ && rag == R_)                   \
    return launch_one<256, 256, AK, BK_, E_, R_>(p, s);
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

}  // namespace moe
