// Tile scheduling and the row-contiguous epilogue shared by the grouped GEMMs.
#pragma once
#include <utility>

#include "common.h"

namespace moe {

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>): compile-time
// indices, whatever the unroller decides (keeps register arrays in registers)
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------ direct-to-LDS stage rings
typedef __attribute__((address_space(3))) void lds_void;
constexpr uint32_t kOOB = 0x80000000u;    // byte offset beyond any buffer extent

// byte offset of 16-byte chunk c (0..7) of row r in a K-contiguous tile of
// 128-byte rows (64 bf16 or 128 fp8 per row): a 16-lane group reading one
// chunk of 16 consecutive rows covers all 64 LDS banks
__device__ __forceinline__ int kc_off(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// raw buffer resource over [base, base + bytes)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7fffffffLL ? 0x7fffffff : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// weight row of fused tile row j (gate rows then up rows per wave column); -1 when beyond f
__device__ __forceinline__ int64_t fused_row(int j, int WN, int64_t n0h, int64_t fdim) {
  const int wc = j / WN, w = j - wc * WN, half = WN >> 1;
  const bool up = w >= half;
  const int64_t col = n0h + wc * half + (up ? w - half : w);
  if (col >= fdim) return -1;
  return up ? fdim + col : col;
}

template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Workgroups are dispatched round-robin over the 8 XCDs (blockIdx % 8). Of
// the `valid` logical tiles, XCD x takes the contiguous run
// [x*valid/8, (x+1)*valid/8): the tiles resident on one XCD at a time share
// A/B panels in that XCD's L2, and every XCD gets the same number of tiles
// to within one, however many surplus workgroups the grid holds (a grouped
// grid is sized for the worst-case tile count). Returns the logical tile of
// this workgroup, or -1 for none. gridDim.x is a multiple of 8 and at least
// valid rounded up to one.
__device__ __forceinline__ int64_t xcd_tile(int64_t valid) {
  const int64_t x = blockIdx.x & 7, i = blockIdx.x >> 3;
  const int64_t lo = x * valid / 8, hi = (x + 1) * valid / 8;
  return lo + i < hi ? lo + i : -1;
}

// Bands of kBandM m-tiles, n-tiles outer inside a band: consecutive logical
// tiles reuse the same B panel across kBandM A panels.
constexpr int kBandM = 8;
__device__ __forceinline__ void band_order(int64_t L, int64_t mt_total, int64_t nt,
                                           int64_t& mt, int64_t& ntile) {
  int64_t band = L / (kBandM * nt);
  int64_t within = L - band * kBandM * nt;
  int64_t rem = mt_total - band * kBandM;
  int64_t h = rem < kBandM ? rem : kBandM;
  mt = band * kBandM + within % h;
  ntile = within / h;
}

// RAG_M tile order: logical tile L lies in group g when
// s_tiles[g] * nt <= L < s_tiles[g+1] * nt, so a group's tiles are
// contiguous and never share a band with another group's. Inside the group,
// local tile u runs band_order over its mtg m-tiles, with the whole group as
// one band when mtg <= kGroupBandMax. Experts with few rows (one or two
// m-tiles) then run all their n-tiles side by side: each weight panel is
// streamed once for both m-tiles and each A panel once for all n-tiles. In
// bands that straddled groups, the tiles resident on an XCD at once read a
// different expert's weight panel per m-tile and re-read the A panels every
// few n-tiles (1.5x the algorithmic HBM traffic on the DeepSeek-like layer).
constexpr int kGroupBandMax = 12;
__device__ __forceinline__ void group_band_order(int64_t u, int64_t mtg, int64_t nt, int64_t& mt,
                                                 int64_t& ntile) {
  if (mtg <= kGroupBandMax) {
    ntile = u / mtg;
    mt = u - ntile * mtg;
  } else {
    band_order(u, mtg, nt, mt, ntile);
  }
}

// Exclusive prefix over groups of ceil(M_g / BM) (M_g from offsets), written
// to s_tiles[0..G] (s_tiles[G] = total; G + 1 ints). 256 threads, G <= 1024.
template <int BM>
__device__ __forceinline__ void group_tile_prefix(const int32_t* __restrict__ off, int G,
                                                  int* s_tiles, int* s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int cnt[4];
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int gi = tid * 4 + i;
    int c = 0;
    if (gi < G) {
      int n = off[gi + 1] - off[gi];
      c = (n + BM - 1) / BM;
    }
    cnt[i] = c;
    s += c;
  }
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wsum[w];
  int ex = base + incl - s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int gi = tid * 4 + i;
    if (gi < G) s_tiles[gi] = ex;
    ex += cnt[i];
  }
  // the total: the last thread's inclusive sum covers all 1024 slots (slots
  // past G count zero), so this also holds for G == 1024
  if (tid == 255) s_tiles[G] = base + incl;
  __syncthreads();
}

// largest g in [0, G) with s_tiles[g] <= mt
__device__ __forceinline__ int find_group(const int* s_tiles, int G, int64_t mt) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_tiles[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Resolved tile of a grouped GEMM.
struct Tile {
  int g;
  int64_t r0;      // first routed row of the group
  int64_t M, K;    // this group's M and K
  int64_t m0, n0;  // tile origin (n0 in output columns; H columns for the fused SwiGLU)
  // tail split-K (RAG_M with GemmArgs::tail_ws): this item computes k-steps
  // [part*ceil(nk/S), ...) of its tile; `slot` indexes the tile's counter
  // (x*cus + j) and its S partials start at item x*cus + j*S. S = 1: whole tile.
  int S = 1, part = 0;
  int64_t slot = 0, item = 0;
};

// Workgroups a RAG_K launch needs (see resolve_tile): 8 * G * ceil(per / 8)
// for per = tiles per group.
inline int64_t rag_k_grid(int64_t G, int64_t per) { return 8 * G * ((per + 7) / 8); }

// Tile `i` of XCD x in a RAG_K launch. The groups' K (their row counts)
// differ, so a group's tiles cost differently from another's. Each group's
// tiles are split into 8 contiguous runs and XCD x takes run x of every
// group, in group order: every XCD does the same share of every group (a
// contiguous split of all tiles would give each XCD whole groups). XCD x
// holds n * G tiles, n = its run length; false when i is past them.
// 32-bit arithmetic: a weight's tile count and an XCD's tile list stay far
// below 2^31 (one expert's weight is under 2 GiB, at most 1024 experts).
template <int BM, int BNo>
__device__ __forceinline__ bool rag_k_tile(const GemmArgs& p, uint32_t x, uint32_t i, Tile& t) {
  const uint32_t nt = (uint32_t)((p.N + BNo - 1) / BNo);
  const uint32_t mtg = (uint32_t)((p.M + BM - 1) / BM);
  const uint32_t per = mtg * nt;
  const uint32_t lo = x * per / 8, n = (x + 1) * per / 8 - lo;
  if (n == 0 || i >= n * (uint32_t)p.G) return false;
  const uint32_t g = i / n, L = lo + (i - g * n);
  // band_order in 32 bits
  const uint32_t band = L / (kBandM * nt);
  const uint32_t within = L - band * kBandM * nt;
  const uint32_t rem = mtg - band * kBandM;
  const uint32_t h = rem < (uint32_t)kBandM ? rem : (uint32_t)kBandM;
  const uint32_t ntile = within / h;
  const uint32_t mt = band * kBandM + (within - ntile * h);
  t.g = (int)g;
  t.m0 = (int64_t)mt * BM;
  t.n0 = (int64_t)ntile * BNo;
  t.M = p.M;
  t.r0 = p.offsets[g];
  t.K = p.offsets[g + 1] - t.r0;
  return true;
}

// Map this workgroup to a tile; false = no tile (surplus workgroup).
// BNo: output columns per tile. s_tiles must hold >= G+1 ints, s_wsum 4 ints.
template <int BM, int BNo, int RAG>
__device__ __forceinline__ bool resolve_tile(const GemmArgs& p, int* s_tiles, int* s_wsum,
                                             Tile& t) {
  const int64_t nt = (p.N + BNo - 1) / BNo;
  if (RAG == RAG_M) {
    group_tile_prefix<BM>(p.offsets, p.G, s_tiles, s_wsum);
    const int64_t total = s_tiles[p.G];
    int64_t L;
    if (p.tail_ws) {
      // XCD x runs its n tiles (the xcd_tile split) on cus CUs: n / cus whole
      // rounds, then r = n mod cus tiles. When r <= cus / 2, each of those r
      // is split into S = min(4, cus / r) parts over K, so the last round
      // runs r*S shorter items instead of r long ones on an idle XCD.
      const int64_t V = total * nt;
      const int64_t x = blockIdx.x & 7, i = blockIdx.x >> 3, cus = p.tail_cus;
      const int64_t lo = x * V / 8, n = (x + 1) * V / 8 - lo;
      const int64_t r = n % cus, full = n - r;
      if (r > 0 && 2 * r <= cus) {
        const int64_t S = cus / r < 4 ? cus / r : 4;
        if (i < full) {
          L = lo + i;
        } else if (i < full + r * S) {
          const int64_t j = (i - full) / S;
          L = lo + full + j;
          t.S = (int)S;
          t.part = (int)((i - full) % S);
          t.slot = x * cus + j;
          t.item = x * cus + j * S;
        } else {
          return false;
        }
      } else {
        if (i >= n) return false;
        L = lo + i;
      }
    } else {
      L = xcd_tile(total * nt);
      if (L < 0) return false;
    }
    t.g = find_group(s_tiles, p.G, L / nt);
    int64_t mt, ntile;
    const int64_t first = s_tiles[t.g];
    group_band_order(L - first * nt, s_tiles[t.g + 1] - first, nt, mt, ntile);
    t.r0 = p.offsets[t.g];
    t.M = p.offsets[t.g + 1] - t.r0;
    t.K = p.K;
    t.m0 = mt * BM;
    t.n0 = ntile * BNo;
    return true;
  }
  // RAG_K: the grid holds 8 * G * ceil(per / 8) workgroups (rag_k_grid);
  // workgroup i of XCD x takes that XCD's tile i
  if (RAG == RAG_K) return rag_k_tile<BM, BNo>(p, blockIdx.x & 7, blockIdx.x >> 3, t);
  const int64_t mtg = (p.M + BM - 1) / BM;
  const int64_t per = mtg * nt;
  const int64_t L = xcd_tile(per * p.G);
  if (L < 0) return false;
  t.g = (int)(L / per);
  int64_t mt, ntile;
  band_order(L - (int64_t)t.g * per, mtg, nt, mt, ntile);
  t.m0 = mt * BM;
  t.n0 = ntile * BNo;
  t.M = p.M;
  t.r0 = (int64_t)t.g * p.M;
  t.K = p.K;
  return true;
}

__device__ __forceinline__ void store1(float* p, float v) { *p = v; }
__device__ __forceinline__ void store1(bf16_t* p, float v) { *p = (bf16_t)f2bf(v); }

template <typename T>
__device__ __forceinline__ const T* operand_base(const Operand& o, const Tile& t) {
  const T* b = reinterpret_cast<const T*>(o.base);
  return o.rowidx ? b + t.r0 * o.ld : b + (int64_t)t.g * o.gstride;
}

// Row-contiguous epilogue over a float32 tile staged in LDS.
// stage[rho * lds + c], rho in [0, nrows), c in [0, ncols) (EPI_SWIGLU_FWD:
// ncols H columns with the gate at c and the up value at ncols + c).
// Stage row rho is output row m0 + rho, stage column c is output column n0 + c.
// Work items are 8-column segments spread over `nthr` threads from `me`.
template <typename TC, int EPI>
__device__ __forceinline__ void epilogue_rows(const GemmArgs& p, const Tile& t, const float* stage,
                                              int lds, int nrows, int ncols, int64_t m0,
                                              int64_t n0, int me, int nthr) {
  TC* cb = reinterpret_cast<TC*>(p.c) + (p.c_rowidx ? t.r0 * p.ldc : (int64_t)t.g * p.c_gstride);
  TC* ab = reinterpret_cast<TC*>(p.aux);
  if (ab) ab += p.aux_rowidx ? t.r0 * p.ldaux : (int64_t)t.g * p.aux_gstride;
  const int segs_per_row = ncols >> 3;
  const int nseg = nrows * segs_per_row;
  for (int s = me; s < nseg; s += nthr) {
    const int rho = s / segs_per_row;
    const int c = (s - rho * segs_per_row) << 3;
    const int64_t gm = m0 + rho, gn = n0 + c;
    if (gm >= t.M || gn >= p.N) continue;
    const float* sv = stage + rho * lds + c;
    float v[8], o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = sv[i];
    if (EPI == EPI_STORE) {
      const int nv = p.N - gn < 8 ? (int)(p.N - gn) : 8;
      if (p.col_bias) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i < nv) v[i] += p.col_bias[gn + i];
      }
      if (nv == 8 && (p.ldc & 7) == 0) {
        Vec8<TC>::store(cb + gm * p.ldc + gn, v);
      } else {
        for (int i = 0; i < nv; ++i) store1(cb + gm * p.ldc + gn + i, v[i]);
      }
    } else if (EPI == EPI_SWIGLU_FWD) {
      float u[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        u[i] = sv[ncols + i];
        o[i] = silu_f(v[i]) * u[i];
      }
      Vec8<TC>::store(cb + gm * p.ldc + gn, o);
      Vec8<TC>::store(ab + gm * p.ldaux + gn, v);
      Vec8<TC>::store(ab + gm * p.ldaux + p.fdim + gn, u);
    } else if (EPI == EPI_GELU_FWD) {
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = gelu_f(v[i]);
      Vec8<TC>::store(cb + gm * p.ldc + gn, o);
      Vec8<TC>::store(ab + gm * p.ldaux + gn, v);
    } else if (EPI == EPI_SWIGLU_BWD) {
      float a[8], b[8], db[8];
      Vec8<TC>::load(ab + gm * p.ldaux + gn, a);
      Vec8<TC>::load(ab + gm * p.ldaux + p.fdim + gn, b);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        o[i] = v[i] * b[i] * dsilu_f(a[i]);
        db[i] = v[i] * silu_f(a[i]);
      }
      Vec8<TC>::store(cb + gm * p.ldc + gn, o);
      Vec8<TC>::store(cb + gm * p.ldc + p.fdim + gn, db);
    } else if (EPI == EPI_GELU_BWD) {
      float a[8];
      Vec8<TC>::load(ab + gm * p.ldaux + gn, a);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = v[i] * dgelu_f(a[i]);
      Vec8<TC>::store(cb + gm * p.ldc + gn, o);
    }
  }
}

}  // namespace moe
