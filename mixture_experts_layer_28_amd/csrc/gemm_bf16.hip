// Grouped GEMM on the bf16 matrix cores of gfx950 (v_mfma_f32_32x32x16_bf16),
// float32 accumulation. One launch covers every expert ("grouped GEMM": each
// expert's GEMM on its own contiguous rows, tiled per expert, one kernel).
//
// Workgroup: 256 threads = 4 waves in a 2x2 grid; tile 256 x 256; each wave
// owns a 128 x 128 sub-tile of 32x32 MFMA blocks whose accumulators fill the
// AGPR file.
//
// Operands stream through a ring of five 32 KiB LDS buffers, each holding one
// operand's 64-k tile (the whole 160 KiB of a CU), filled by
// buffer_load ... lds (global -> LDS with no staging registers). A
// K-contiguous operand row is 128 bytes of global memory, a whole cache line:
// measured on gfx950, DMA of 128-byte row pieces feeds a CU about 1.65x
// faster than 64-byte pieces. Operand X of k-step k lives in buffer
// (2k + X) mod 5 (A = 0, B = 1), so each tile reuses the buffer of the one
// five places earlier in the sequence A0 B0 A1 B1 ...; B tiles are loaded one
// k-step ahead and A tiles two, one DMA instruction per four MFMAs.
// Per k-step (4 slices of 16 k, 16 MFMAs each, with the next slice's
// fragments read between the MFMAs of the current one):
//   slice 0: the second half of B_{kt+1};
//   slices 1, 2: A_{kt+2};
//   wait for A_{kt+1} and B_{kt+1} (A_{kt+2} may stay in flight), barrier:
//   every read of A_kt and B_kt has been issued and waited for;
//   slice 3: reads k-step kt+1's slice-0 fragments and issues the first half
//   of B_{kt+2} into A_kt's buffer.
// Five k-steps per loop trip name their buffers statically; the last
// nk mod 5 k-steps run after the loop (exits inside the unrolled trip made
// the register allocator spill).
//
// LDS layouts (bank-conflict free for the fragment reads):
//   K-contiguous operand, [rows][64] bf16 (128-byte rows): 16-byte chunk c of
//     row r at r*128 + ((c ^ ((r >> 1) & 7)) << 4); a 16-lane group reading
//     one chunk of 16 consecutive rows then covers all 64 banks.
//   K-strided operand (the transposed reads of the backward), [64][rows]:
//     16-byte slot s (8 rows) of k-row k at k*rows*2 + ((s ^ ((k & 3) << 1)) << 4);
//     fragments are built by ds_read_b64_tr_b16, which transposes 4x4
//     blocks of bf16 across each 16-lane group.
// A DMA instruction fills a contiguous 1 KiB with lane l at byte 16*l, so a
// layout's swizzle is realised by choosing the global chunk each lane fetches.
// Lanes that fall outside the operand (ragged rows, the K tail, k-steps past
// the end) point past the buffer's extent and read zeros.
#include "gemm_tile.h"

namespace moe {

constexpr int kBK = 64;                   // k per operand tile
constexpr int kRows = 256;                // tile rows of either operand

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

// 8 floats -> 8 bf16 at p (16-byte aligned), one nontemporal 16-byte store.
// Every epilogue output (H, the saved pre-activations, dpre, C) is written
// once and not read again by the launch, so it streams past the caches.
__device__ __forceinline__ void store8_nt(bf16_t* p, const float* v) {
  v4u32 u;
  u[0] = pack_bf2(v[0], v[1]); u[1] = pack_bf2(v[2], v[3]);
  u[2] = pack_bf2(v[4], v[5]); u[3] = pack_bf2(v[6], v[7]);
  __builtin_nontemporal_store(u, reinterpret_cast<v4u32*>(p));
}

// byte offset of slot s (rows 8s..8s+7) of k-row k in a K-strided [64][kRows] tile
__device__ __forceinline__ int ks_off(int k, int s) {
  return k * (kRows * 2) + ((s ^ ((k & 3) << 1)) << 4);
}


struct DmaSrc {
  uint32_t off[8];
  int kk[8];
};

// Per-lane DMA source of one operand tile: a wave issues 8 instructions per
// tile; instruction i fills 1 KiB block blk = wave*8 + i. off[i] is the byte
// offset at k0 = 0 (kOOB when the rows lie outside the operand); kk[i] is the
// lane's k inside the tile, for the K-tail test.
//   K-contiguous: block = rows blk*8 .. +7 (128 bytes each), lane l -> row
//     blk*8 + (l>>3), physical chunk l&7, logical chunk (l&7) ^ ((row>>1)&7).
//   K-strided: block = k-rows 2*blk, 2*blk+1, lane l -> k-row 2*blk + (l>>5),
//     logical slot (l&31) ^ ((k&3)<<1), i.e. rows 8*slot .. 8*slot+7.
template <bool KC, bool FUSED, int WN>
__device__ __forceinline__ void dma_src(DmaSrc& d, int64_t ld, int64_t rows_valid, int64_t r0,
                                        int64_t fdim, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int blk = wave * 8 + i;
    if (KC) {
      const int r = blk * 8 + (lane >> 3);
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
      d.off[i] = ok ? (uint32_t)((grow * ld + c * 8) * 2) : kOOB;
      d.kk[i] = c * 8;
    } else {
      const int k = blk * 2 + (lane >> 5);
      const int s = (lane & 31) ^ ((k & 3) << 1);
      const int64_t grow = r0 + s * 8;
      d.off[i] = grow < rows_valid ? (uint32_t)((k * ld + grow) * 2) : kOOB;
      d.kk[i] = k;
    }
  }
}

__device__ __forceinline__ void unpack8_bf16(uint4 w, float* v) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = bf2f(u[e] & 0xffffu);
    v[2 * e + 1] = bf2f(u[e] >> 16);
  }
}


__device__ __forceinline__ bf16x8 join(v4i16 lo, v4i16 hi) {
  const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

template <int EPI, bool AKM, bool BKM, int RAG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int BM = kRows, BN = kRows;
  constexpr int WM = BM / 2, WN = BN / 2, MI = WM / 32, NI = WN / 32, NM = MI * NI;
  constexpr bool FUSED = EPI == EPI_SWIGLU_FWD;
  constexpr int BNo = FUSED ? BN / 2 : BN;      // output columns per tile
  constexpr int A_EL = BM * kBK, B_EL = BN * kBK;   // elements per operand tile
  static_assert(A_EL == B_EL, "ring buffers hold either operand");
  static_assert(!FUSED || BKM, "fused SwiGLU needs a K-contiguous weight");
  static_assert(NM == 16 && MI + NI == 8, "schedule assumes 4x4 MFMA blocks per wave");
  // Five 32 KiB buffers, each holding one operand's 64-k tile; separate
  // objects so that the compiler can tell a buffer being filled from one read.
  __shared__ __attribute__((aligned(1024))) bf16_t h0[A_EL];
  __shared__ __attribute__((aligned(1024))) bf16_t h1[A_EL];
  __shared__ __attribute__((aligned(1024))) bf16_t h2[A_EL];
  __shared__ __attribute__((aligned(1024))) bf16_t h3[A_EL];
  __shared__ __attribute__((aligned(1024))) bf16_t h4[A_EL];

  Tile t;
  {
    // the group-tile scan runs before any load and borrows the last stage
    int* s_tiles = reinterpret_cast<int*>(h4);
    const bool have = resolve_tile<BM, BNo, RAG>(p, s_tiles, s_tiles + 1028, t);
    __syncthreads();
    if (!have) return;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
  // buffer extents: K-contiguous operands span rows x ld, K-strided span K x ld
  const int64_t b_rows = FUSED ? 2 * p.fdim : p.N;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(operand_base<bf16_t>(p.a, t), (AKM ? t.M : t.K) * p.a.ld * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(operand_base<bf16_t>(p.b, t), (BKM ? b_rows : t.K) * p.b.ld * 2);
  DmaSrc da, db;
  dma_src<AKM, false, WN>(da, p.a.ld, t.M, t.m0, p.fdim, wave, lane);
  dma_src<BKM, FUSED, WN>(db, p.b.ld, FUSED ? p.fdim : p.N, t.n0, p.fdim, wave, lane);

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // k-steps of this tile; a tail split-K item takes its part of them
  constexpr bool TAIL = EPI == EPI_STORE && RAG == RAG_M;
  int64_t nk = (t.K + kBK - 1) / kBK;
  int64_t kbase = 0;
  if (TAIL && t.S > 1) {
    const int64_t per = (nk + t.S - 1) / t.S;
    kbase = per * t.part;
    nk = kbase >= nk ? 0 : (nk - kbase < per ? nk - kbase : per);
  }

  // DMA instruction i (0..7) of operand X (0 = A, 1 = B) of k-step kt into buffer s
  auto dma = [&](int64_t kt, int X, bf16_t* s, int i) __attribute__((always_inline)) {
    const int64_t k0 = (kbase + kt) * kBK;
    const bool isA = X == 0;
    const DmaSrc& d = isA ? da : db;
    const bool kc = isA ? AKM : BKM;
    const int64_t ld = isA ? p.a.ld : p.b.ld;
    const bool kin = d.kk[i] < t.K - k0;
    const uint32_t so = (uint32_t)(kc ? k0 * 2 : k0 * ld * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? ra : rb, (lds_void*)(s + (wave * 8 + i) * 512), 16,
                                             kin ? d.off[i] : kOOB, so, 0, 0);
  };

  // K-strided fragments (ds_read_b64_tr_b16). Block qq of a wave's rows
  // (rows w0 + 32qq .. +31, w0 = wm0 or wn0) for k slice sl: lane (g, i) =
  // (lane >> 4, lane & 15) reads row w0 + 32qq + 16(g & 1) + 4(i & 3) at k-rows
  // k and k + 4, k = 16sl + 8(g >> 1) + (i >> 2). In the [64][256] layout
  // (ks_off) that byte offset splits into a lane part, which depends on qq only
  // through its parity, and a compile-time part:
  //   ks_off(k, row >> 3) + 2(row & 7) = tlo[qq & 1] + 8192 sl + 64 (qq & ~1)
  //   (+ 2048 for k + 4), with
  //   tlo[par] = 512 kl + 2 w0 + 64 (par ^ xb) + 16 (y ^ (x & 3)) + 2 (rl & 7),
  // kl = 8(g >> 1) + (i >> 2), rl = 16(g & 1) + 4(i & 3), x = (kl & 3) << 1,
  // y = rl >> 3, xb = x >> 2. So every read is one of two lane offsets per
  // operand plus an immediate, instead of an address register per read.
  auto tr_lane_off = [&](int w0, int par) __attribute__((always_inline)) -> int {
    const int g = lane >> 4, i = lane & 15;
    const int rl = 16 * (g & 1) + 4 * (i & 3), kl = 8 * (g >> 1) + (i >> 2);
    const int x = (kl & 3) << 1, y = rl >> 3, xb = x >> 2;
    return 512 * kl + 2 * w0 + 64 * (par ^ xb) + 16 * (y ^ (x & 3)) + 2 * (rl & 7);
  };
  const int tlo_a[2] = {tr_lane_off(wm0, 0), tr_lane_off(wm0, 1)};
  const int tlo_b[2] = {tr_lane_off(wn0, 0), tr_lane_off(wn0, 1)};

  // fragment of block qq (rows w0 + 32qq .. +31) for k slice sl (0..3) of an operand tile
  auto frag = [&](const bf16_t* tile, bool kc, bool isA, int qq, int sl) __attribute__((always_inline)) -> bf16x8 {
    const char* tb = reinterpret_cast<const char*>(tile);
    if (kc)
      return *reinterpret_cast<const bf16x8*>(
          tb + kc_off((isA ? wm0 : wn0) + qq * 32 + (lane & 31), sl * 2 + (lane >> 5)));
    const char* lb = tb + (isA ? tlo_a[qq & 1] : tlo_b[qq & 1]) + 8192 * sl + 64 * (qq & ~1);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)lb);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lb + 2048));
    return join(lo, hi);
  };

  bf16x8 fa0[MI], fb0[NI], fa1[MI], fb1[NI];
  auto ldfrag_q = [&](bf16x8* fa, bf16x8* fb, const bf16_t* sa, const bf16_t* sb, int sl, int q)
      __attribute__((always_inline)) {
    if (q < MI) fa[q] = frag(sa, AKM, true, q, sl);
    else fb[q - MI] = frag(sb, BKM, false, q - MI, sl);
  };
  auto mma = [&](const bf16x8* fa, const bf16x8* fb, int q) __attribute__((always_inline)) {
    const int i = q / NI, j = q % NI;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  };

  // 16 MFMAs on (fa, fb), reading slice rsl of (rsa, rsb) into (ga, gb)
  // between them, and DMA instructions i0 .. i0+3 of operand X of k-step dk
  // into buffer ds (one per four MFMAs)
  auto slice = [&](const bf16x8* fa, const bf16x8* fb, bf16x8* ga, bf16x8* gb, const bf16_t* rsa,
                   const bf16_t* rsb, int rsl, int64_t dk, int X, bf16_t* ds, int i0)
      __attribute__((always_inline)) {
    static_for<NM>([&](auto Q) __attribute__((always_inline)) {
      constexpr int q = decltype(Q)::value;
      mma(fa, fb, q);
      __builtin_amdgcn_sched_barrier(0);
      if (q < MI + NI) ldfrag_q(ga, gb, rsa, rsb, rsl, q);
      if ((q & 3) == 3) dma(dk, X, ds, i0 + (q >> 2));
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Buffer of operand X of k-step k: (2k + X) mod 5, so an operand tile reuses
  // the buffer of the one five places earlier in the sequence A0 B0 A1 B1 ...
  // k-step kt (its slice-0 fragments already in fa0/fb0; A_{kt+1} and the
  // first half of B_{kt+1} in flight since the previous k-step):
  //   slice 0: second half of B_{kt+1} (into A_{kt-1}'s old buffer);
  //   slices 1, 2: A_{kt+2} (into B_{kt-1}'s old buffer);
  //   wait for A_{kt+1}, B_{kt+1} (only A_{kt+2} may stay in flight), barrier:
  //   every read of A_kt and B_kt is done;
  //   slice 3: reads k-step kt+1's slice-0 fragments and issues the first half
  //   of B_{kt+2} into A_kt's buffer.
  // B tiles have one k-step to land, A tiles two; one DMA per four MFMAs.
  auto kstep = [&](int64_t kt, bf16_t* a0, bf16_t* b0, bf16_t* a1, bf16_t* b1, bf16_t* a2,
                   bf16_t* b2) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    slice(fa0, fb0, fa1, fb1, a0, b0, 1, kt + 1, 1, b1, 4);
    slice(fa1, fb1, fa0, fb0, a0, b0, 2, kt + 2, 0, a2, 0);
    slice(fa0, fb0, fa1, fb1, a0, b0, 3, kt + 2, 0, a2, 4);
    wait_vm<8>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    slice(fa1, fb1, fa0, fb0, a1, b1, 0, kt + 2, 1, b2, 0);
  };

  // as if just after the barrier of k-step -1: A0, B0, A1 and half of B1
  // (28 DMA instructions per wave)
  auto prologue = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) dma(0, 0, h0, i);
#pragma unroll
    for (int i = 0; i < 8; ++i) dma(0, 1, h1, i);
#pragma unroll
    for (int i = 0; i < 8; ++i) dma(1, 0, h2, i);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma(1, 1, h3, i);
  };
  // the k-steps of the tile, A0 and B0 landed and visible to every wave
  auto mainloop = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < MI + NI; ++q) ldfrag_q(fa0, fb0, h0, h1, 0, q);
    // five k-steps per trip name their buffers statically; the trip stops at
    // the last k-step (loads past the end read zeros and are waited for below)
    int64_t kt = 0;
    for (; kt + 5 <= nk; kt += 5) {
      kstep(kt, h0, h1, h2, h3, h4, h0);
      kstep(kt + 1, h2, h3, h4, h0, h1, h2);
      kstep(kt + 2, h4, h0, h1, h2, h3, h4);
      kstep(kt + 3, h1, h2, h3, h4, h0, h1);
      kstep(kt + 4, h3, h4, h0, h1, h2, h3);
    }
    // the last nk mod 5 k-steps (buffer phase continues from 0)
    if (kt < nk) kstep(kt, h0, h1, h2, h3, h4, h0);
    if (kt + 1 < nk) kstep(kt + 1, h2, h3, h4, h0, h1, h2);
    if (kt + 2 < nk) kstep(kt + 2, h4, h0, h1, h2, h3, h4);
    if (kt + 3 < nk) kstep(kt + 3, h1, h2, h3, h4, h0, h1);
  };


  if (nk > 0) {
    prologue();
    wait_vm<12>();
    __builtin_amdgcn_s_barrier();
    mainloop();
    wait_vm<0>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
  }

  if constexpr (TAIL) {
    if (t.S > 1) {
      // Tail split-K: store this item's fp32 accumulators ([register][thread]),
      // count the tile's arrived items; the last to arrive adds the S partials
      // in part order (the same sum whichever arrives last) and stores the tile.
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
      // per 16-register block, all four parts' values are loaded before any
      // is added (parts past S read part S-1 and count as zero), then added
      // in part order
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

  // ---- epilogue: per 32-row block row i, the wave stages its 32 x 128 fp32
  // results in a stage of its own (one 16-byte write per (j, g): the four
  // consecutive columns the transposed accumulators hold), then reads them
  // back row-contiguous, two adjacent 16-byte slots (8 columns) per lane, and
  // stores 16 bytes of bf16 per lane per output. Slot s of staged row r sits
  // at r*512 + ((s ^ (r & 7)) << 4); the two rows a 16-lane group reads take
  // slots of opposite parity, so the readback is conflict-free.
  // N and every leading dimension are multiples of 8, so an 8-column segment
  // is wholly inside or wholly outside the output.
  char* stg = reinterpret_cast<char*>(wave < 2 ? h0 : h1) + (wave & 1) * 16384;
  bf16_t* cb = reinterpret_cast<bf16_t*>(p.c) + (p.c_rowidx ? t.r0 * p.ldc : (int64_t)t.g * p.c_gstride);
  bf16_t* ab = reinterpret_cast<bf16_t*>(p.aux);
  if (ab) ab += p.aux_rowidx ? t.r0 * p.ldaux : (int64_t)t.g * p.aux_gstride;
  const int lr = lane & 31, lh = lane >> 5;
  // plain / GELU / backward epilogues: lane l takes slots 2s, 2s+1 (s = l&15)
  // of row 4q + (l>>4), q = 0..7
  const int s8 = lane & 15, rq = lane >> 4;
  const int64_t n8 = t.n0 + wn0 + 8 * s8;
  // Backward epilogues read this lane's saved pre-activations (a, and b for
  // SwiGLU) of each block row: the loads of block row i+1 are issued when
  // block row i starts, so they overlap its staging, math and stores
  // (rows/columns clamped into range when out).
  constexpr bool BWD = EPI == EPI_SWIGLU_BWD || EPI == EPI_GELU_BWD;
  constexpr bool SW = EPI == EPI_SWIGLU_BWD;
  uint4 pa[2][BWD ? 8 : 1], pb[2][SW ? 8 : 1];
  auto aux_load = [&](int ii, uint4* da_, uint4* db_) __attribute__((always_inline)) {
    const int64_t nc = n8 < p.N ? n8 : p.N - 8;
    static_for<8>([&](auto Q) __attribute__((always_inline)) {
      constexpr int q = decltype(Q)::value;
      int64_t m = t.m0 + wm0 + 32 * ii + 4 * q + rq;
      m = m < t.M ? m : t.M - 1;
      da_[q] = *reinterpret_cast<const uint4*>(ab + m * p.ldaux + nc);
      if (SW) db_[q] = *reinterpret_cast<const uint4*>(ab + m * p.ldaux + p.fdim + nc);
    });
  };
  if (BWD) aux_load(0, pa[0], pb[0]);
  if (EPI == EPI_STORE) {
    // plain store: the output is bf16, so the block row is staged as bf16
    // (half the LDS traffic of float32 staging, same bits). Row r of the
    // block row is 256 bytes at r*256; its 16-byte slot s (columns 8s..8s+7)
    // sits at ((s ^ (r & 15)) << 4), so the 32 rows a (j, g) write touches
    // spread over all banks and a 16-lane group's row readback is a
    // permutation of one row. Lane (lr, lh) holds columns 32j + 8g + 4lh .. +3:
    // slot 4j + g, 8-byte half lh. The output is written once and not read
    // again by this launch, so its stores are nontemporal (streamed past the
    // caches): a weight gradient with K = 256 spends about 2.6 us of a 15 us
    // tile issuing its 128 KiB of stores, and nontemporal ones take 1 us off.
    static_for<MI>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      static_for<NI * 4>([&](auto Q) __attribute__((always_inline)) {
        constexpr int j = decltype(Q)::value / 4, g = decltype(Q)::value % 4;
        uint2 w;
        w.x = pack_bf2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
        w.y = pack_bf2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        *reinterpret_cast<uint2*>(stg + lr * 256 + (((4 * j + g) ^ (lr & 15)) << 4) + 8 * lh) = w;
      });
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_wave_barrier();
      const int64_t mrow0 = t.m0 + wm0 + 32 * i;
      const bool nok = n8 < p.N;
      static_for<8>([&](auto Q) __attribute__((always_inline)) {
        constexpr int q = decltype(Q)::value;
        const int r = 4 * q + rq;
        const uint4 u = *reinterpret_cast<const uint4*>(stg + r * 256 + ((s8 ^ (r & 15)) << 4));
        const int64_t m = mrow0 + r;
        if (m < t.M && nok)
          __builtin_nontemporal_store(__builtin_bit_cast(v4u32, u), reinterpret_cast<v4u32*>(cb + m * p.ldc + n8));
      });
      // the next block row overwrites the stage: finish this one's reads;
      // and keep its accumulator reads and conversions here (hoisted ahead,
      // they would hold all 128 packed registers at once)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_sched_barrier(0);
    });
    return;
  }
  static_for<MI>([&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    if (BWD && i + 1 < MI) aux_load(i + 1, pa[(i + 1) & 1], pb[(i + 1) & 1]);
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
    auto ld8 = [&](int r, int slot, float* v) __attribute__((always_inline)) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(stg + r * 512 + ((slot ^ (r & 7)) << 4));
      const f32x4 y = *reinterpret_cast<const f32x4*>(stg + r * 512 + (((slot + 1) ^ (r & 7)) << 4));
      v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
      v[4] = y[0]; v[5] = y[1]; v[6] = y[2]; v[7] = y[3];
    };
    if (EPI == EPI_SWIGLU_FWD) {
      // slots 0..15 hold gate columns, 16..31 the matching up columns: lane l
      // takes gate slots 2(l&7), +1 and the up slots 16 above them, of row
      // 8q + (l>>3), q = 0..3
      const int sg = lane & 7, rr = lane >> 3;
      const int64_t hc = t.n0 + (wave & 1) * (WN / 2) + 8 * sg;
      static_for<4>([&](auto Q) __attribute__((always_inline)) {
        constexpr int q = decltype(Q)::value;
        const int r = 8 * q + rr;
        float a[8], b[8], h[8];
        ld8(r, 2 * sg, a);
        ld8(r, 16 + 2 * sg, b);
        const int64_t m = mrow0 + r;
        if (m >= t.M || hc >= p.N) return;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = silu_f(a[e]) * b[e];
        store8_nt(cb + m * p.ldc + hc, h);
        store8_nt(ab + m * p.ldaux + hc, a);
        store8_nt(ab + m * p.ldaux + p.fdim + hc, b);
      });
    } else {
      const bool nok = n8 < p.N;
      const uint4* ra = pa[i & 1];
      const uint4* rb = pb[i & 1];
      static_for<8>([&](auto Q) __attribute__((always_inline)) {
        constexpr int q = decltype(Q)::value;
        const int r = 4 * q + rq;
        float v[8], o[8];
        ld8(r, 2 * s8, v);
        const int64_t m = mrow0 + r;
        if (m >= t.M || !nok) return;
        if (EPI == EPI_STORE) {
          store8_nt(cb + m * p.ldc + n8, v);
        } else if (EPI == EPI_STORE_F32) {
          // float32 partial products, read back at once by the fold kernel:
          // ordinary (cached) stores
          float* cf = reinterpret_cast<float*>(p.c) +
                      (p.c_rowidx ? t.r0 * p.ldc : (int64_t)t.g * p.c_gstride) + m * p.ldc + n8;
          f32x4 lo4, hi4;
          lo4[0] = v[0]; lo4[1] = v[1]; lo4[2] = v[2]; lo4[3] = v[3];
          hi4[0] = v[4]; hi4[1] = v[5]; hi4[2] = v[6]; hi4[3] = v[7];
          *reinterpret_cast<f32x4*>(cf) = lo4;
          *reinterpret_cast<f32x4*>(cf + 4) = hi4;
        } else if (EPI == EPI_GELU_FWD) {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = gelu_f(v[e]);
          store8_nt(cb + m * p.ldc + n8, o);
          store8_nt(ab + m * p.ldaux + n8, v);
        } else {
          float a[8];
          unpack8_bf16(ra[BWD ? q : 0], a);
          if (SW) {
            float b[8], o2[8];
            unpack8_bf16(rb[SW ? q : 0], b);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              o[e] = v[e] * b[e] * dsilu_f(a[e]);
              o2[e] = v[e] * silu_f(a[e]);
            }
            store8_nt(cb + m * p.ldc + n8, o);
            store8_nt(cb + m * p.ldc + p.fdim + n8, o2);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = v[e] * dgelu_f(a[e]);
            store8_nt(cb + m * p.ldc + n8, o);
          }
        }
      });
    }
    // the next block row overwrites the stage: finish this one's reads
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
  });
}

// ------------------------------------------------------------------ launch
template <bool AKM, bool BKM, int EPI, int RAG>
static hipError_t launch_one(const GemmArgs& p, hipStream_t s) {
  constexpr int BNo = EPI == EPI_SWIGLU_FWD ? kRows / 2 : kRows;
  const int64_t nt = (p.N + BNo - 1) / BNo;
  int64_t tiles;
  if (RAG == RAG_M)
    tiles = ((p.max_rows + kRows - 1) / kRows + p.G) * nt;
  else
    tiles = (int64_t)p.G * ((p.M + kRows - 1) / kRows) * nt;
  int64_t nb = RAG == RAG_K ? rag_k_grid(p.G, ((p.M + kRows - 1) / kRows) * nt)
                            : (tiles + 7) / 8 * 8;
  // tail split-K: up to tail_cus more items per XCD
  if (RAG == RAG_M && EPI == EPI_STORE && p.tail_ws) nb += 8 * (int64_t)p.tail_cus;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<EPI, AKM, BKM, RAG>), dim3((unsigned)nb), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Dispatch over the layouts/epilogues the layer uses.
hipError_t gemm_bf16(const GemmArgs& p, bool akm, bool bkm, int epi, int rag, hipStream_t s) {
  if (p.col_bias) return hipErrorInvalidValue;   // column bias is an fp32-GEMM feature only
#define MOE_CASE(AK, BK_, E_, R_)                                          \
  if (akm == AK && bkm == BK_ && epi == E_ && rag == R_)                   \
    return launch_one<AK, BK_, E_, R_>(p, s);
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
  MOE_CASE(true, true, EPI_STORE_F32, RAG_NONE)
  MOE_CASE(true, false, EPI_STORE_F32, RAG_NONE)
  MOE_CASE(false, false, EPI_STORE_F32, RAG_NONE)
#undef MOE_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
