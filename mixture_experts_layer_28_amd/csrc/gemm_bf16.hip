// Grouped GEMM on the bf16 matrix cores of gfx950 (v_mfma_f32_32x32x16_bf16),
// float32 accumulation. One launch covers every expert ("grouped GEMM": each
// expert's GEMM on its own contiguous rows, tiled per expert, one kernel).
//
// Workgroup: 256 threads = 4 waves in a 2x2 grid; tile BM x BN x 64; each
// wave owns a (BM/2) x (BN/2) sub-tile of 32x32 MFMA blocks whose
// accumulators live in the AGPR file.
//
// LDS holds both operands K-contiguous ([rows][64] bf16 = 128 B per row) in
// two stages. Each 16-byte chunk c of row r sits at position
// c ^ (r & 7) ^ ((r >> 3) & 7): the fragment reads (32 consecutive rows, one
// chunk), the row-wise stores (one row, all chunks) and the transposed
// stores (8 rows 8 apart, one chunk) all spread over every bank.
//
// A K-contiguous operand is copied global -> LDS by buffer_load ... lds
// (no staging registers, no LDS store instructions); lane l of a wave
// instruction lands at LDS byte 16*l of that instruction's 1 KiB block, so the
// swizzle is realised by choosing which global chunk each lane fetches.
// Out-of-range lanes (ragged rows, K tail) point past the buffer's extent and
// read zeros. A K-strided operand (the transposed reads of the backward) goes
// through registers: 8x8 blocks loaded row-wise, transposed in registers,
// stored as K-contiguous chunks.
//
// Per k-step the next stage's loads are issued first, then the MFMAs run on
// the current stage with the fragments of k-slice s+1 read from LDS while the
// MFMAs of slice s execute.
#include "gemm_tile.h"

namespace moe {

constexpr int kBK = 64;
constexpr uint32_t kOOB = 0x80000000u;   // byte offset beyond any buffer extent

__device__ __forceinline__ int swz_pos(int row, int chunk) {
  return chunk ^ (row & 7) ^ ((row >> 3) & 7);
}
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kBK + (swz_pos(row, chunk) << 3);
}

// raw buffer resource over [base, base + bytes)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7fffffffLL ? 0x7fffffff : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

typedef __attribute__((address_space(3))) void lds_void;

// weight row of fused tile row j; -1 when beyond f
__device__ __forceinline__ int64_t fused_row(int j, int WN, int64_t n0h, int64_t fdim) {
  const int wc = j / WN, w = j - wc * WN, half = WN >> 1;
  const bool up = w >= half;
  const int64_t col = n0h + wc * half + (up ? w - half : w);
  if (col >= fdim) return -1;
  return up ? fdim + col : col;
}

// ---- K-contiguous operand: global -> LDS directly.
// The tile has ROWS rows of 8 chunks; ROWS/8 blocks of 1 KiB; each of the 4
// waves issues ROWS/32 instructions.
template <int ROWS, bool FUSED, int WN>
__device__ __forceinline__ void direct_load(__amdgpu_buffer_rsrc_t rs, bf16_t* lds_tile, int64_t ld,
                                            int64_t rows_valid, int64_t r0, int64_t k0, int64_t K,
                                            int64_t fdim, int wave_u, int lane) {
#pragma unroll
  for (int i = 0; i < ROWS / 32; ++i) {
    const int blk = wave_u * (ROWS / 32) + i;
    const int r = blk * 8 + (lane >> 3);
    const int c = (lane & 7) ^ (lane >> 3) ^ (blk & 7);
    int64_t grow;
    bool ok;
    if (FUSED) {
      grow = fused_row(r, WN, r0, fdim);
      ok = grow >= 0;
    } else {
      grow = r0 + r;
      ok = grow < rows_valid;
    }
    const int64_t kk = k0 + c * 8;
    ok = ok && kk < K;
    const uint32_t off = ok ? (uint32_t)((grow * ld + kk) * 2) : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds_tile + blk * 512), 16, off, 0, 0, 0);
  }
}

// ---- K-strided operand: element (row, kk) at base + kk*ld + row.
template <int ROWS>
struct Strided {
  static constexpr int NIT = (ROWS + 255) / 256;
  uint4 r[NIT * 8];
};

template <int ROWS>
__device__ __forceinline__ void strided_load(Strided<ROWS>& L, __amdgpu_buffer_rsrc_t rs, int64_t ld,
                                             int64_t rows_valid, int64_t r0, int64_t k0, int64_t K) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < Strided<ROWS>::NIT; ++it) {
    const int q = tid + 256 * it;
    const int kb = q / (ROWS / 8), mb = q - kb * (ROWS / 8);
    const int64_t grow = r0 + mb * 8;
    const bool okq = q < ROWS && grow < rows_valid;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int64_t kk = k0 + kb * 8 + rr;
      const uint32_t off = (okq && kk < K) ? (uint32_t)((kk * ld + grow) * 2) : kOOB;
      L.r[it * 8 + rr] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    }
  }
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

template <int ROWS>
__device__ __forceinline__ void strided_store(const Strided<ROWS>& L, bf16_t* lds) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < Strided<ROWS>::NIT; ++it) {
    const int q = tid + 256 * it;
    if (q >= ROWS) continue;
    const int kb = q / (ROWS / 8), mb = q - kb * (ROWS / 8);
    const uint4* R = &L.r[it * 8];
    // R[rr] holds k = kb*8+rr for rows mb*8 .. mb*8+7 (two rows per dword)
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

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int BM, int BN, bool AKM, bool BKM, int EPI, int RAG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2, MI = WM / 32, NI = WN / 32;
  constexpr bool FUSED = EPI == EPI_SWIGLU_FWD;
  constexpr int BNo = FUSED ? BN / 2 : BN;      // output columns per tile
  constexpr int A_EL = BM * kBK, B_EL = BN * kBK;
  constexpr int BUF = A_EL + B_EL;              // one stage: A tile then B tile
  constexpr int LDST = WN + 4;                  // staging row stride (floats)
  static_assert(2 * 32 * LDST * 4 <= BUF * 2, "staging does not fit");
  static_assert(!FUSED || BKM, "fused SwiGLU needs a K-contiguous weight");
  // The two stages are separate objects so that the compiler can tell the
  // stage being filled by direct loads from the stage being read (it would
  // otherwise wait for every in-flight load before each LDS read).
  __shared__ __attribute__((aligned(1024))) bf16_t lds0[BUF];
  __shared__ __attribute__((aligned(1024))) bf16_t lds1[BUF];
  __shared__ int s_tiles[1028];
  __shared__ int s_wsum[4];

  Tile t;
  if (!resolve_tile<BM, BNo, RAG>(p, s_tiles, s_wsum, t)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
  const bf16_t* Ab = operand_base<bf16_t>(p.a, t);
  const bf16_t* Bb = operand_base<bf16_t>(p.b, t);
  const int64_t b_rows = FUSED ? p.fdim : p.N;
  // buffer extents: K-contiguous operands span rows x ld, K-strided span K x ld
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(Ab, (AKM ? t.M : t.K) * p.a.ld * 2);
  const __amdgpu_buffer_rsrc_t rb =
      make_rsrc(Bb, (BKM ? (FUSED ? 2 * p.fdim : p.N) : t.K) * p.b.ld * 2);

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  Strided<BM> sa;
  Strided<BN> sb;
  const int64_t nk = (t.K + kBK - 1) / kBK;

  auto issue = [&](int64_t kt, bf16_t* as) __attribute__((always_inline)) {
    const int64_t k0 = kt * kBK;
    if (AKM) direct_load<BM, false, WN>(ra, as, p.a.ld, t.M, t.m0, k0, t.K, p.fdim, wave, lane);
    else strided_load<BM>(sa, ra, p.a.ld, t.M, t.m0, k0, t.K);
    if (BKM) direct_load<BN, FUSED, WN>(rb, as + A_EL, p.b.ld, b_rows, t.n0, k0, t.K, p.fdim, wave, lane);
    else strided_load<BN>(sb, rb, p.b.ld, p.N, t.n0, k0, t.K);
  };
  auto finish = [&](bf16_t* as) __attribute__((always_inline)) {
    if (!AKM) strided_store<BM>(sa, as);
    if (!BKM) strided_store<BN>(sb, as + A_EL);
  };
  // one k-step: loads of tile kt+1 into `nxt` (for kt+1 == nk every lane is
  // out of range and zeros land in the idle stage), MFMAs on `cur`
  auto kstep = [&](int64_t kt, const bf16_t* cur, bf16_t* nxt) __attribute__((always_inline)) {
    issue(kt + 1, nxt);
    const bf16_t* as = cur;
    const bf16_t* bs = cur + A_EL;
    bf16x8 fa[2][MI], fb[2][NI];
    auto ldfrag = [&](int buf, int kk) __attribute__((always_inline)) {
      const int ch = kk * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < MI; ++i)
        fa[buf][i] = *reinterpret_cast<const bf16x8*>(as + swz(wm0 + i * 32 + (lane & 31), ch));
#pragma unroll
      for (int j = 0; j < NI; ++j)
        fb[buf][j] = *reinterpret_cast<const bf16x8*>(bs + swz(wn0 + j * 32 + (lane & 31), ch));
    };
    ldfrag(0, 0);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      // one scheduling region per slice: the next slice's fragment reads are
      // issued, then this slice's MFMAs run while they are in flight
      __builtin_amdgcn_sched_barrier(0);
      if (kk + 1 < kBK / 16) ldfrag((kk + 1) & 1, kk + 1);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][i], fb[kk & 1][j],
                                                              acc[i][j], 0, 0, 0);
      if (kk + 1 < kBK / 16) {
        // start the reads early: one after each of the first MI+NI MFMAs
#pragma unroll
        for (int x = 0; x < MI + NI; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, MI * NI - (MI + NI), 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    finish(nxt);
    wait_vm_all();
    __syncthreads();
  };

  if (nk > 0) {
    issue(0, lds0);
    finish(lds0);
    wait_vm_all();
    __syncthreads();
  }
  // two k-steps per trip, so each names its stages statically; for odd nk
  // the last step multiplies the all-zero stage left by out-of-range loads
  for (int64_t kt = 0; kt < nk; kt += 2) {
    kstep(kt, lds0, lds1);
    kstep(kt + 1, lds1, lds0);
  }

  // ---- epilogue: stage 32 rows of the wave's sub-tile at a time in LDS
  // (waves 0-1 in the first stage's space, waves 2-3 in the second's)
  float* stage = reinterpret_cast<float*>(wave < 2 ? lds0 : lds1) + (wave & 1) * (32 * LDST);
  static_for<MI>([&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
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
    else if (EPI == EPI_SWIGLU_BWD || EPI == EPI_GELU_BWD)
      epilogue_act_bwd<(EPI == EPI_SWIGLU_BWD ? EPI_SWIGLU_BWD : EPI_GELU_BWD), 32, WN, 64>(
          p, t, stage, LDST, m0, t.n0 + wn0, lane);
    else
      epilogue_rows<bf16_t, EPI>(p, t, stage, LDST, 32, WN, m0, t.n0 + wn0, lane, 64);
    __syncthreads();
  });
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
