// Grouped GEMM on FP8 (OCP E4M3) operands on the gfx950 matrix cores
// (v_mfma_f32_32x32x64_f8f6f4, float32 accumulation), for the forward of the
// expert FFN and the backward's data gradients (whose weight operand is the
// transposed weight, quantized per input channel, or in square blocks with
// block scales below). Both operands are
// K-contiguous byte matrices with one
// power-of-two scale per row (2^a_sexp[m] for the input rows, 2^b_sexp[n]
// for the weight rows); the epilogue applies them exactly with ldexp, so
//   C[m][n] = 2^(a_sexp[m] + b_sexp[n]) * sum_k e4m3(A[m][k]) e4m3(B[n][k]).
//
// Workgroup: 256 threads = 4 waves in a 2x2 grid; tile 256 x 256; each wave
// owns 128 x 128 as 4 x 4 MFMA blocks of 32 x 32 held in AGPRs.
//
// LDS is a ring of five 32 KiB buffers, each holding one operand's 128-k
// tile: 256 rows x 128 bytes, whole 128-byte lines per DMA row piece, in the
// bf16 GEMM's layout (chunk c of row r at r*128 + ((c ^ ((r >> 1) & 7)) << 4),
// 16 fp8 per chunk). Operand X of k-step k (A = 0, B = 1) lives in buffer
// (2k + X) mod 5, reusing the buffer of the tile five places earlier in the
// sequence A0 B0 A1 B1 .... A k-step is two slices of 64 k, one MFMA per
// 32 x 32 block each. The matrix core takes from lane l (row l & 31, half
// h = l >> 5) 32 bytes: k 16h .. 16h+15 of its 64-k slice in the first 16
// bytes and k 32+16h .. 32+16h+15 in the next 16 (measured on gfx950), so a
// fragment of slice sl is chunks 4sl+h and 4sl+2+h of its row.
// Per k-step: slice 0 (slice 1's fragments read between the MFMAs; A_{kt+2}
// issued into B_{kt-1}'s old buffer); wait for A_{kt+1} and B_{kt+1}
// (A_{kt+2} may stay in flight), barrier (every read of A_kt and B_kt is
// done); slice 1 (k-step kt+1's slice-0 fragments read; B_{kt+2} issued into
// A_kt's buffer). A tiles have three slices to land, B tiles two; one DMA
// instruction per two MFMAs.
//
// Block scales (BLK, GemmArgs::blk_scales): instead of one exponent per row,
// one 8-bit exponent (e8m0: e + 127) per 32 elements along K of every row of
// either operand, applied inside the matrix instruction by its block-scaled
// form (v_mfma_scale_f32_32x32x64_f8f6f4): lane l supplies the exponent of
// row l & 31 for the 32-k block l >> 5 of its 64-k slice. A row's 4 bytes of
// a 128-k step form one 32-bit word, and the words of 32 consecutive rows for
// one k-step are contiguous (32-row interleaved layout), so the load of a
// 32-row block's words touches one or two 128-byte lines (a row-major layout
// made it 32 lines and slowed the loop by about 45%). Each lane loads its
// rows' words for the next k-step with the current one's DMAs and shifts them
// right by 8 (l >> 5), so byte 2 sl holds its block of slice sl. The epilogue
// then applies no exponent.
#include "gemm_tile.h"

namespace moe {

namespace {

constexpr int kBK8 = 128;                 // k per operand tile (bytes per tile row)
constexpr int kRows8 = 256;               // tile rows of either operand

typedef int v8i32 __attribute__((ext_vector_type(8)));

struct Dma8 {
  uint32_t off[8];
  int kk[8];
};

// Per-lane DMA source: instruction i of a wave fills 1 KiB block
// blk = wave*8 + i = rows blk*8 .. +7 (128 bytes each); lane l -> row
// blk*8 + (l >> 3), physical chunk l & 7, logical chunk (l & 7) ^ ((row >> 1) & 7).
template <bool FUSED, int WN>
__device__ __forceinline__ void dma_src8(Dma8& d, int64_t ld, int64_t rows_valid, int64_t r0,
                                         int64_t fdim, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (wave * 8 + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    int64_t grow;
    bool ok;
    if (FUSED) {
      grow = fused_row(r, WN, r0, fdim);
      ok = grow >= 0;
    } else {
      grow = r0 + r;
      ok = grow < rows_valid;
    }
    d.off[i] = ok ? (uint32_t)(grow * ld + c * 16) : kOOB;
    d.kk[i] = c * 16;
  }
}


__device__ __forceinline__ void unpack8(uint4 w, float* v) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = bf2f(u[e] & 0xffffu);
    v[2 * e + 1] = bf2f(u[e] >> 16);
  }
}

__device__ __forceinline__ v8i32 join8(int4 lo, int4 hi) {
  v8i32 v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

// AF: the FP8 format of the A operand (0 = E4M3, 1 = E5M2: the backward's
// gradient rows); B is always E4M3
template <int EPI, int RAG, bool BLK, int AF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_fp8_kernel(GemmArgs p) {
  constexpr int BM = kRows8, BN = kRows8;
  constexpr int WM = BM / 2, WN = BN / 2, MI = WM / 32, NI = WN / 32, NM = MI * NI;
  constexpr bool FUSED = EPI == EPI_SWIGLU_FWD;
  constexpr int BNo = FUSED ? BN / 2 : BN;
  constexpr int A_B = BM * kBK8, B_B = BN * kBK8;   // bytes per operand tile
  static_assert(A_B == B_B, "ring buffers hold either operand");
  static_assert(NM == 16 && MI + NI == 8, "schedule assumes 4x4 MFMA blocks per wave");
  __shared__ __attribute__((aligned(1024))) char h0[A_B];
  __shared__ __attribute__((aligned(1024))) char h1[A_B];
  __shared__ __attribute__((aligned(1024))) char h2[A_B];
  __shared__ __attribute__((aligned(1024))) char h3[A_B];
  __shared__ __attribute__((aligned(1024))) char h4[A_B];

  Tile t;
  {
    int* s_tiles = reinterpret_cast<int*>(h4);
    const bool have = resolve_tile<BM, BNo, RAG>(p, s_tiles, s_tiles + 1028, t);
    __syncthreads();
    if (!have) return;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
  const uint8_t* Ab = operand_base<uint8_t>(p.a, t);
  const uint8_t* Bb = operand_base<uint8_t>(p.b, t);
  const int64_t b_rows = FUSED ? 2 * p.fdim : p.N;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab, t.M * p.a.ld);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb, b_rows * p.b.ld);
  Dma8 da, db;
  dma_src8<false, WN>(da, p.a.ld, t.M, t.m0, p.fdim, wave, lane);
  dma_src8<FUSED, WN>(db, p.b.ld, FUSED ? p.fdim : p.N, t.n0, p.fdim, wave, lane);

  // block scales (32-row interleaved words: word w of row r at
  // (r / 32 * KW + w) * 32 + r % 32): the k-step-0 word offset of each of
  // this lane's rows, by matrix row (A: the group's first row + m; B: group
  // g's b_sexp_gstride rows + n). Rows outside are clamped into range: they
  // read zero codes, so any exponent does.
  // RAG_K (weight gradients): both operands are token-axis transposes
  // ([rows, Rp] codes, Rp = the row stride) in which group g's tokens start
  // at k = kpos = 128 * (ceil(r0 / 128) + g); their scale rows hold Rp / 128
  // words and the group's words start at kpos / 128.
  const int64_t KW = (t.K + kBK8 - 1) / kBK8;
  const int64_t kpos = RAG == RAG_K ? kBK8 * ((t.r0 + kBK8 - 1) / kBK8 + t.g) : 0;
  const int64_t KWrow = RAG == RAG_K ? p.a.ld / kBK8 : KW;
  const uint32_t* swa = reinterpret_cast<const uint32_t*>(p.a_sexp);
  const uint32_t* swb = reinterpret_cast<const uint32_t*>(p.b_sexp);
  auto word0 = [&](int64_t r) __attribute__((always_inline)) {
    return (uint32_t)(((r >> 5) * KWrow) * 32 + (r & 31));
  };
  // Per lane, the word of its block-0 row and how many of its 32-row blocks
  // lie inside the operand: block i's row is 32 i below block 0's, so its
  // word is 32 i * KWrow further on; blocks past the operand read a fixed
  // in-range row's word (A: the last row, B: the group's first). A few VALU
  // operations per load instead of one register per block. The fused SwiGLU
  // B rows (gate and up halves) keep one offset per block.
  const uint32_t KW32 = (uint32_t)(KWrow * 32);
  uint32_t sa_w0 = 0, sa_last = 0, sb_w0 = 0, sb_last = 0;
  int sa_nv = 0, sb_nv = 0;
  uint32_t sb_off[BLK && FUSED ? NI : 1];
  uint32_t sa_nxt[BLK ? MI : 1], sb_nxt[BLK ? NI : 1], sa_cur[BLK ? MI : 1], sb_cur[BLK ? NI : 1];
  if constexpr (BLK) {
    const int64_t arow0 = RAG == RAG_K ? 0 : (p.a.rowidx ? t.r0 : (int64_t)t.g * p.M);
    const int64_t m0l = t.m0 + wm0 + (lane & 31);
    sa_w0 = word0(arow0 + m0l);
    sa_last = word0(arow0 + t.M - 1);
    sa_nv = m0l < t.M ? (int)((t.M - m0l + 31) / 32) : 0;
    const int64_t brow0 = (int64_t)t.g * p.b_sexp_gstride;
    if constexpr (FUSED) {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int64_t n = fused_row(wn0 + 32 * j + (lane & 31), WN, t.n0, p.fdim);
        sb_off[j] = word0(brow0 + (n < 0 ? 0 : n));
      }
    } else {
      const int64_t n0l = t.n0 + wn0 + (lane & 31);
      sb_w0 = word0(brow0 + n0l);
      sb_last = word0(brow0);
      sb_nv = n0l < p.N ? (int)((p.N - n0l + 31) / 32) : 0;
    }
  }

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // k-steps of this tile; a tail split-K item takes its part of them
  constexpr bool TAIL = EPI == EPI_STORE && RAG == RAG_M;
  int64_t nk = (t.K + kBK8 - 1) / kBK8;
  int64_t kbase = 0;
  if (TAIL && t.S > 1) {
    const int64_t per = (nk + t.S - 1) / t.S;
    kbase = per * t.part;
    nk = kbase >= nk ? 0 : (nk - kbase < per ? nk - kbase : per);
  }
  // BLK: words of k-step kt into the nxt registers (k-steps past the end
  // read the last word: their codes are zero); nxt -> cur, shifted
  auto load_scales = [&](int64_t kt) __attribute__((always_inline)) {
    if constexpr (BLK) {
      const int64_t kg0 = kbase + kt;
      const uint32_t kg = 32 * (uint32_t)(kpos / kBK8 + (kg0 < KW ? kg0 : KW - 1));
#pragma unroll
      for (int i = 0; i < MI; ++i) sa_nxt[i] = swa[(i < sa_nv ? sa_w0 + i * KW32 : sa_last) + kg];
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        uint32_t o;
        if constexpr (FUSED) o = sb_off[j];
        else o = j < sb_nv ? sb_w0 + j * KW32 : sb_last;
        sb_nxt[j] = swb[o + kg];
      }
    }
  };
  auto take_scales = [&]() __attribute__((always_inline)) {
    if constexpr (BLK) {
      const int sh = 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < MI; ++i) sa_cur[i] = sa_nxt[i] >> sh;
#pragma unroll
      for (int j = 0; j < NI; ++j) sb_cur[j] = sb_nxt[j] >> sh;
    }
  };

  // DMA instruction i (0..7) of operand X (0 = A, 1 = B) of k-step kt into buffer s
  auto dma = [&](int64_t kt, int X, char* s, int i) __attribute__((always_inline)) {
    const int64_t k0 = (kbase + kt) * kBK8;
    const Dma8& d = X == 0 ? da : db;
    const bool kin = d.kk[i] < t.K - k0;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(X == 0 ? ra : rb, (lds_void*)(s + (wave * 8 + i) * 1024), 16,
                                             kin ? d.off[i] : kOOB, (uint32_t)(kpos + k0), 0, 0);
  };

  // half `part` of the fragment of rows base .. base+31 for slice sl
  auto frag = [&](const char* tile, int base, int sl, int part) __attribute__((always_inline)) -> int4 {
    return *reinterpret_cast<const int4*>(tile + kc_off(base + (lane & 31), 4 * sl + 2 * part + (lane >> 5)));
  };

  int4 xa[MI][2], xb[NI][2], ya[MI][2], yb[NI][2];
  // read half `part` of fragment q (0..3: A blocks, 4..7: B blocks) of slice sl of (sa, sb)
  auto ldfrag = [&](int4 (*fa)[2], int4 (*fb)[2], const char* sa, const char* sb, int sl, int q,
                    int part) __attribute__((always_inline)) {
    if (q < MI) fa[q][part] = frag(sa, wm0 + q * 32, sl, part);
    else fb[q - MI][part] = frag(sb, wn0 + (q - MI) * 32, sl, part);
  };
  // Transposed accumulation (B fragment first): lane l holds row
  // wm0+32i+(l&31) and, in acc[i][j][4g..4g+3], columns wn0+32j+8g+4(l>>5)+0..3.
  // Constant zero scale operands select the unscaled instruction (scale 1).
  // BLK: the first operand (B rows) takes sb_cur[j], the second (A rows)
  // sa_cur[i]; byte 2 sl of the shifted word is the lane's 32-k block of
  // slice sl
  auto mma = [&](int4 (*fa)[2], int4 (*fb)[2], int q, auto SL) __attribute__((always_inline)) {
    const int i = q / NI, j = q % NI;
    if constexpr (BLK) {
      constexpr int os = 2 * decltype(SL)::value;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          join8(fb[j][0], fb[j][1]), join8(fa[i][0], fa[i][1]), acc[i][j], 0, AF, os, (int)sb_cur[j], os,
          (int)sa_cur[i]);
    } else {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          join8(fb[j][0], fb[j][1]), join8(fa[i][0], fa[i][1]), acc[i][j], 0, AF, 0, 0, 0, 0);
    }
  };

  // 16 MFMAs on (fa, fb), reading slice rsl of (rsa, rsb) into (ga, gb)
  // between them and issuing operand X of k-step dk into ds, one DMA per two
  auto slice = [&](int4 (*fa)[2], int4 (*fb)[2], int4 (*ga)[2], int4 (*gb)[2], const char* rsa,
                   const char* rsb, int rsl, int64_t dk, int X, char* ds, auto SL) __attribute__((always_inline)) {
    static_for<NM>([&](auto Q) __attribute__((always_inline)) {
      constexpr int q = decltype(Q)::value;
      mma(fa, fb, q, SL);
      __builtin_amdgcn_sched_barrier(0);
      ldfrag(ga, gb, rsa, rsb, rsl, q >> 1, q & 1);
      if (q & 1) dma(dk, X, ds, q >> 1);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // BLK: k-step kt's scale words (loaded during k-step kt-1) become the
  // current ones, and k-step kt+1's are loaded before this k-step's DMAs, so
  // the wait below (only A_{kt+2} in flight) also covers them
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  auto kstep = [&](int64_t kt, char* a0, char* b0, char* a1, char* b1, char* a2, char* b2)
      __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    take_scales();
    load_scales(kt + 1);
    slice(xa, xb, ya, yb, a0, b0, 1, kt + 2, 0, a2, S0{});
    wait_vm<8>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    slice(ya, yb, xa, xb, a1, b1, 0, kt + 2, 1, b2, S1{});
  };

  if (nk > 0) {
    // as if just before k-step 0: A0, B0 (and k-step 0's scale words) landed,
    // A1 and B1 in flight
    load_scales(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) dma(0, 0, h0, i);
#pragma unroll
    for (int i = 0; i < 8; ++i) dma(0, 1, h1, i);
#pragma unroll
    for (int i = 0; i < 8; ++i) dma(1, 0, h2, i);
#pragma unroll
    for (int i = 0; i < 8; ++i) dma(1, 1, h3, i);
    wait_vm<16>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int q = 0; q < MI + NI; ++q) {
      ldfrag(xa, xb, h0, h1, 0, q, 0);
      ldfrag(xa, xb, h0, h1, 0, q, 1);
    }
    // five k-steps per trip name their buffers statically; the last nk mod 5
    // k-steps run after the loop (loads past the end read zeros)
    int64_t kt = 0;
    for (; kt + 5 <= nk; kt += 5) {
      kstep(kt, h0, h1, h2, h3, h4, h0);
      kstep(kt + 1, h2, h3, h4, h0, h1, h2);
      kstep(kt + 2, h4, h0, h1, h2, h3, h4);
      kstep(kt + 3, h1, h2, h3, h4, h0, h1);
      kstep(kt + 4, h3, h4, h0, h1, h2, h3);
    }
    if (kt < nk) kstep(kt, h0, h1, h2, h3, h4, h0);
    if (kt + 1 < nk) kstep(kt + 1, h2, h3, h4, h0, h1, h2);
    if (kt + 2 < nk) kstep(kt + 2, h4, h0, h1, h2, h3, h4);
    if (kt + 3 < nk) kstep(kt + 3, h1, h2, h3, h4, h0, h1);
    wait_vm<0>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
  }

  if constexpr (TAIL) {
    if (t.S > 1) {
      // Tail split-K, as in the bf16 GEMM: store this item's fp32
      // accumulators ([register][thread]), count the tile's arrived items;
      // the last adds the S partials in part order and stores the tile (the
      // per-row exponents apply to the sum as to a whole tile's accumulators).
      char* tw = reinterpret_cast<char*>(p.tail_ws);
      float* parts = reinterpret_cast<float*>(tw + tail_counter_bytes(p.tail_cus));
      float* mine = parts + (t.item + t.part) * 65536;
      static_for<MI * NI>([&](auto Q) __attribute__((always_inline)) {
        constexpr int q = decltype(Q)::value;
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[(q * 16 + r) * 256 + tid] = acc[q / NI][q % NI][r];
      });
      __threadfence();
      __syncthreads();
      int* last = reinterpret_cast<int*>(h4);   // the ring is idle now; stages use h0, h1
      if (tid == 0) {
        const int old = __hip_atomic_fetch_add(reinterpret_cast<int*>(tw) + t.slot, 1,
                                               __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        *last = old == t.S - 1;
      }
      __syncthreads();
      if (!*last) return;
      __threadfence();
      const float* all = parts + t.item * 65536;
      const int S = t.S;
      static_for<MI * NI>([&](auto Q) __attribute__((always_inline)) {
        constexpr int q = decltype(Q)::value;
        float w[4][16];
#pragma unroll
        for (int sp = 0; sp < 4; ++sp)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            w[sp][r] = all[(int64_t)(sp < S ? sp : S - 1) * 65536 + (q * 16 + r) * 256 + tid];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = w[0][r];
          v += S > 1 ? w[1][r] : 0.f;
          v += S > 2 ? w[2][r] : 0.f;
          v += S > 3 ? w[3][r] : 0.f;
          acc[q / NI][q % NI][r] = v;
        }
      });
    }
  }

  // ---- epilogue: stage each 32-row block row in fp32 (a stage per wave),
  // read it back row-contiguous 8 columns per lane, scale by
  // 2^(a_sexp + b_sexp), store 16 bytes of bf16 per lane per output.
  // Slot s of staged row r sits at r*512 + ((s ^ (r & 7)) << 4); the two rows
  // a 16-lane group reads take slots of opposite parity (conflict-free).
  char* stg = (wave < 2 ? h0 : h1) + (wave & 1) * 16384;
  bf16_t* cb = reinterpret_cast<bf16_t*>(p.c) + (p.c_rowidx ? t.r0 * p.ldc : (int64_t)t.g * p.c_gstride);
  bf16_t* ab = reinterpret_cast<bf16_t*>(p.aux);
  if (ab) ab += p.aux_rowidx ? t.r0 * p.ldaux : (int64_t)t.g * p.aux_gstride;
  const int32_t* asx = p.a_sexp + (p.a.rowidx ? t.r0 : (int64_t)t.g * p.M);
  const int32_t* bsx = p.b_sexp + (int64_t)t.g * p.b_sexp_gstride;
  const int lr = lane & 31, lh = lane >> 5;
  // Backward epilogues: this lane's saved pre-activations (a, and b for
  // SwiGLU) of the block row are loaded before its accumulators are staged,
  // so the loads overlap the staging (rows/columns clamped into range).
  constexpr bool BWD = EPI == EPI_SWIGLU_BWD || EPI == EPI_GELU_BWD;
  constexpr bool SW = EPI == EPI_SWIGLU_BWD;
  static_for<MI>([&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    uint4 pa8[BWD ? 8 : 1], pb8[SW ? 8 : 1];
    if (BWD) {
      const int64_t n = t.n0 + wn0 + 8 * (lane & 15);
      const int64_t nc = n < p.N ? n : p.N - 8;
      static_for<8>([&](auto Q) __attribute__((always_inline)) {
        constexpr int q = decltype(Q)::value;
        int64_t m = t.m0 + wm0 + 32 * i + 4 * q + (lane >> 4);
        m = m < t.M ? m : t.M - 1;
        pa8[BWD ? q : 0] = *reinterpret_cast<const uint4*>(ab + m * p.ldaux + nc);
        if (SW) pb8[SW ? q : 0] = *reinterpret_cast<const uint4*>(ab + m * p.ldaux + p.fdim + nc);
      });
    }
    static_for<NI * 4>([&](auto Q) __attribute__((always_inline)) {
      constexpr int j = decltype(Q)::value / 4, g = decltype(Q)::value % 4;
      const int sl = 8 * j + 2 * g + lh;
      f32x4 v;
      v[0] = acc[i][j][4 * g];
      v[1] = acc[i][j][4 * g + 1];
      v[2] = acc[i][j][4 * g + 2];
      v[3] = acc[i][j][4 * g + 3];
      *reinterpret_cast<f32x4*>(stg + lr * 512 + ((sl ^ (lr & 7)) << 4)) = v;
    });
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    const int64_t mrow0 = t.m0 + wm0 + 32 * i;
    // lane lr holds the scale exponent of row mrow0 + lr (clamped into range)
    const int64_t mcl = mrow0 + lr < t.M ? mrow0 + lr : t.M - 1;
    const int ea_l = BLK ? 0 : asx[mcl];
    // 8 consecutive staged columns (slots slot, slot+1) of row r
    auto ld8 = [&](int r, int slot, float* v) __attribute__((always_inline)) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(stg + r * 512 + ((slot ^ (r & 7)) << 4));
      const f32x4 y = *reinterpret_cast<const f32x4*>(stg + r * 512 + (((slot + 1) ^ (r & 7)) << 4));
      v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
      v[4] = y[0]; v[5] = y[1]; v[6] = y[2]; v[7] = y[3];
    };
    auto ld_exp8 = [&](const int32_t* e, int* out) __attribute__((always_inline)) {
      const int4 x = *reinterpret_cast<const int4*>(e);
      const int4 y = *reinterpret_cast<const int4*>(e + 4);
      out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
      out[4] = y.x; out[5] = y.y; out[6] = y.z; out[7] = y.w;
    };
    if (EPI == EPI_SWIGLU_FWD) {
      // lane l: gate slots 2(l&7), +1 and the up slots 16 above, of row 8q + (l>>3)
      const int sg = lane & 7, rr = lane >> 3;
      const int64_t hc = t.n0 + (wave & 1) * (WN / 2) + 8 * sg;
      const int64_t hcl = hc < p.N ? hc : p.N - 8;
      int egs[8] = {0, 0, 0, 0, 0, 0, 0, 0}, eus[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (!BLK) {
        ld_exp8(bsx + hcl, egs);
        ld_exp8(bsx + p.fdim + hcl, eus);
      }
      static_for<4>([&](auto Q) __attribute__((always_inline)) {
        constexpr int q = decltype(Q)::value;
        const int r = 8 * q + rr;
        const int ea = __shfl(ea_l, r, 64);
        float a[8], b[8], h[8];
        ld8(r, 2 * sg, a);
        ld8(r, 16 + 2 * sg, b);
        const int64_t m = mrow0 + r;
        if (m >= t.M || hc >= p.N) return;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          a[e] = ldexpf(a[e], ea + egs[e]);
          b[e] = ldexpf(b[e], ea + eus[e]);
          h[e] = silu_f(a[e]) * b[e];
        }
        Vec8<bf16_t>::store(cb + m * p.ldc + hc, h);
        Vec8<bf16_t>::store(ab + m * p.ldaux + hc, a);
        Vec8<bf16_t>::store(ab + m * p.ldaux + p.fdim + hc, b);
      });
    } else {
      // lane l: slots 2(l&15), +1 of row 4q + (l>>4)
      const int s8 = lane & 15, rq = lane >> 4;
      const int64_t n = t.n0 + wn0 + 8 * s8;
      const bool nok = n < p.N;
      int ebs[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (!BLK) ld_exp8(bsx + (nok ? n : p.N - 8), ebs);
      static_for<8>([&](auto Q) __attribute__((always_inline)) {
        constexpr int q = decltype(Q)::value;
        const int r = 4 * q + rq;
        const int ea = __shfl(ea_l, r, 64);
        float v[8], o[8];
        ld8(r, 2 * s8, v);
        const int64_t m = mrow0 + r;
        if (m >= t.M || !nok) return;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = ldexpf(v[e], ea + ebs[e]);
        if (EPI == EPI_STORE) {
          Vec8<bf16_t>::store(cb + m * p.ldc + n, v);
        } else if (EPI == EPI_GELU_FWD) {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = gelu_f(v[e]);
          Vec8<bf16_t>::store(cb + m * p.ldc + n, o);
          Vec8<bf16_t>::store(ab + m * p.ldaux + n, v);
        } else {
          // v = dH; C = dpre = [da | db] (SwiGLU) or da (GELU)
          float a[8];
          unpack8(pa8[BWD ? q : 0], a);
          if (SW) {
            float b[8], o2[8];
            unpack8(pb8[SW ? q : 0], b);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              o[e] = v[e] * b[e] * dsilu_f(a[e]);
              o2[e] = v[e] * silu_f(a[e]);
            }
            Vec8<bf16_t>::store(cb + m * p.ldc + n, o);
            Vec8<bf16_t>::store(cb + m * p.ldc + p.fdim + n, o2);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = v[e] * dgelu_f(a[e]);
            Vec8<bf16_t>::store(cb + m * p.ldc + n, o);
          }
        }
      });
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
  });
}

template <int EPI, int RAG, bool BLK, int AF = 0>
hipError_t launch_fp8(const GemmArgs& p, hipStream_t s) {
  constexpr int BNo = EPI == EPI_SWIGLU_FWD ? kRows8 / 2 : kRows8;
  const int64_t nt = (p.N + BNo - 1) / BNo;
  int64_t tiles;
  if (RAG == RAG_M)
    tiles = ((p.max_rows + kRows8 - 1) / kRows8 + p.G) * nt;
  else
    tiles = (int64_t)p.G * ((p.M + kRows8 - 1) / kRows8) * nt;
  int64_t nb = (tiles + 7) / 8 * 8;
  if (RAG == RAG_K) nb = rag_k_grid(p.G, ((p.M + kRows8 - 1) / kRows8) * nt);
  // tail split-K: up to tail_cus more items per XCD
  if (RAG == RAG_M && EPI == EPI_STORE && p.tail_ws) nb += 8 * (int64_t)p.tail_cus;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_fp8_kernel<EPI, RAG, BLK, AF>), dim3((unsigned)nb), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

// FP8 grouped GEMM, both operands K-contiguous (the forward's layouts, and
// the data gradients against transposed weights). With block scales also
// RAG_K: the weight gradients, both operands token-axis transposes with each
// group's tokens from k = 128 * (ceil(offsets[g] / 128) + g) (groups may hold
// any number of rows; the codes past a group's rows within its last k-step
// must be zero).
// Requires K % 16 == 0 (RAG_M, RAG_NONE), 16-byte aligned rows, N % 4 == 0
// (f % 4 for the fused SwiGLU) and 16-byte aligned scale arrays; the caller
// checks.
hipError_t gemm_fp8(const GemmArgs& p, int epi, int rag, hipStream_t s, int a_fmt) {
  if (!p.a_sexp || !p.b_sexp || p.col_bias || a_fmt < 0 || a_fmt > 1) return hipErrorInvalidValue;
#define MOE_CASE(E_, R_) \
  if (epi == E_ && rag == R_) return launch_fp8<E_, R_, false>(p, s);
#define MOE_CASE_BLK(E_, R_) \
  if (epi == E_ && rag == R_) return launch_fp8<E_, R_, true>(p, s);
#define MOE_CASE_A5(E_, R_, B_) \
  if (epi == E_ && rag == R_ && (bool)p.blk_scales == B_) return launch_fp8<E_, R_, B_, 1>(p, s);
  if (a_fmt == 1) {
    // E5M2 A operand: the backward's gradient rows (data gradients against
    // the transposed weights, per-row or block scales) and the weight
    // gradients' token-axis gradient operand (block scales)
    MOE_CASE_A5(EPI_SWIGLU_BWD, RAG_M, false)
    MOE_CASE_A5(EPI_GELU_BWD, RAG_M, false)
    MOE_CASE_A5(EPI_STORE, RAG_M, false)
    MOE_CASE_A5(EPI_SWIGLU_BWD, RAG_NONE, false)
    MOE_CASE_A5(EPI_GELU_BWD, RAG_NONE, false)
    MOE_CASE_A5(EPI_STORE, RAG_NONE, false)
    MOE_CASE_A5(EPI_SWIGLU_BWD, RAG_M, true)
    MOE_CASE_A5(EPI_GELU_BWD, RAG_M, true)
    MOE_CASE_A5(EPI_STORE, RAG_M, true)
    MOE_CASE_A5(EPI_SWIGLU_BWD, RAG_NONE, true)
    MOE_CASE_A5(EPI_GELU_BWD, RAG_NONE, true)
    MOE_CASE_A5(EPI_STORE, RAG_NONE, true)
    MOE_CASE_A5(EPI_STORE, RAG_K, true)
    return hipErrorInvalidValue;
  }
  if (p.blk_scales) {
    // block scales: the forward GEMMs, the data gradients (dH with the
    // activation backward, dX as a plain store)
    MOE_CASE_BLK(EPI_SWIGLU_FWD, RAG_M)
    MOE_CASE_BLK(EPI_GELU_FWD, RAG_M)
    MOE_CASE_BLK(EPI_STORE, RAG_M)
    MOE_CASE_BLK(EPI_SWIGLU_FWD, RAG_NONE)
    MOE_CASE_BLK(EPI_GELU_FWD, RAG_NONE)
    MOE_CASE_BLK(EPI_STORE, RAG_NONE)
    MOE_CASE_BLK(EPI_SWIGLU_BWD, RAG_M)
    MOE_CASE_BLK(EPI_GELU_BWD, RAG_M)
    MOE_CASE_BLK(EPI_SWIGLU_BWD, RAG_NONE)
    MOE_CASE_BLK(EPI_GELU_BWD, RAG_NONE)
    // and the weight gradients on token-axis transposes
    MOE_CASE_BLK(EPI_STORE, RAG_K)
    return hipErrorInvalidValue;
  }
  MOE_CASE(EPI_SWIGLU_FWD, RAG_M)
  MOE_CASE(EPI_GELU_FWD, RAG_M)
  MOE_CASE(EPI_STORE, RAG_M)
  MOE_CASE(EPI_SWIGLU_BWD, RAG_M)
  MOE_CASE(EPI_GELU_BWD, RAG_M)
  MOE_CASE(EPI_SWIGLU_FWD, RAG_NONE)
  MOE_CASE(EPI_GELU_FWD, RAG_NONE)
  MOE_CASE(EPI_STORE, RAG_NONE)
  MOE_CASE(EPI_SWIGLU_BWD, RAG_NONE)
  MOE_CASE(EPI_GELU_BWD, RAG_NONE)
#undef MOE_CASE
#undef MOE_CASE_BLK
#undef MOE_CASE_A5
  return hipErrorInvalidValue;
}

}  // namespace moe
