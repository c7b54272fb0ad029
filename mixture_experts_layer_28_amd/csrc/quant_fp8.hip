// Per-row FP8 (OCP E4M3) quantization with power-of-two scales, the input
// side of the FP8 forward GEMMs. Row i of a bf16 matrix becomes
//   codes[i][k] = E4M3 nearest (ties to even) of x[i][k] * 2^-e_i,
// e_i = the smallest integer with max_k |x[i][k]| <= 448 * 2^e_i (0 for an
// all-zero row). Multiplying by a power of two is exact, so the conversion
// instruction's rounding is the only rounding; the codes are a bit-exact
// function of the input. Inputs must be finite. The per-row and token-axis
// quantizers also write OCP E5M2 (the backward's gradient operands, largest
// magnitude 1.75 * 2^15 in place of 448).
//
// One workgroup of 256 threads per row; each thread keeps up to eight
// 16-byte chunks of its row in registers between the max pass and the
// conversion pass (rows up to 16384 wide), longer rows are read twice.
//
// The transposing form quantizes each column of a row-major matrix as a row
// of its transpose (the backward reads the weights along their input
// dimension): a column-max pass, then a 64 x 64 tiled transpose.
#include "common.h"

namespace moe {

namespace {

constexpr int kQThreads = 256;
constexpr int kQCache = 8;   // 16-byte chunks a thread keeps in registers

// eight bf16 scaled by 2^-e -> eight E4M3 codes (byte i = element i)
__device__ __forceinline__ uint2 to_e4m3(uint4 v, int e) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float a = ldexpf(bf2f(w[2 * h] & 0xffffu), -e);
    const float b = ldexpf(bf2f(w[2 * h] >> 16), -e);
    const float c = ldexpf(bf2f(w[2 * h + 1] & 0xffffu), -e);
    const float d = ldexpf(bf2f(w[2 * h + 1] >> 16), -e);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    o[h] = (uint32_t)r;
  }
  return make_uint2(o[0], o[1]);
}

template <int FMT>
__global__ __launch_bounds__(kQThreads) void quant_rows_fp8_kernel(
    const bf16_t* __restrict__ src, int64_t K, int64_t ld_src, const int32_t* __restrict__ valid_rows,
    uint8_t* __restrict__ codes, int64_t ld_q, int32_t* __restrict__ sexp) {
  const int64_t row = blockIdx.x;
  if (valid_rows && row >= (int64_t)*valid_rows) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint4* s = reinterpret_cast<const uint4*>(src + row * ld_src);
  uint2* q = reinterpret_cast<uint2*>(codes + row * ld_q);
  const int64_t nch = K / 8;
  uint4 cache[kQCache];
  uint32_t m = 0;
#pragma unroll
  for (int u = 0; u < kQCache; ++u) {
    const int64_t c = tid + (int64_t)u * kQThreads;
    cache[u] = c < nch ? s[c] : make_uint4(0, 0, 0, 0);
    m = absmax8(cache[u], m);
  }
  for (int64_t c = tid + (int64_t)kQCache * kQThreads; c < nch; c += kQThreads) m = absmax8(s[c], m);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t t = __shfl_xor(m, o, 64);
    m = t > m ? t : m;
  }
  __shared__ uint32_t wmax[kQThreads / 64];
  if (lane == 0) wmax[wave] = m;
  __syncthreads();
  m = wmax[0];
#pragma unroll
  for (int w = 1; w < kQThreads / 64; ++w) m = wmax[w] > m ? wmax[w] : m;
  // e: amax = mant * 2^ex (mant in [0.5, 1)); amax <= 1.75 * 2^(8 + e)
  const int e = fp8_scale_exp<FMT>(m, bf2f(m));
  if (tid == 0) sexp[row] = e;
#pragma unroll
  for (int u = 0; u < kQCache; ++u) {
    const int64_t c = tid + (int64_t)u * kQThreads;
    if (c < nch) q[c] = to_fp8<FMT>(cache[u], e);
  }
  for (int64_t c = tid + (int64_t)kQCache * kQThreads; c < nch; c += kQThreads) q[c] = to_fp8<FMT>(s[c], e);
}

// ---- block scales: one exponent per 32 elements along K
// Row r, block b (elements 32b .. 32b+31, the last one partial when K is not
// a multiple of 32): e = the per-row rule on the block's maximum, clipped to
// [-127, 127]; codes as above; the exponent is stored as the byte e + 127.
// Layout (32-row interleaved): the four bytes of blocks 4w .. 4w+3 of a row
// form 32-bit word w (w < KW = ceil(K / 128); blocks past K hold 127), and
// word w of rows 32g .. 32g+31 sits at words (g * KW + w) * 32 + (r & 31), so
// the GEMM reads one k-step's words of 32 consecutive rows as one 128-byte
// line. One thread per 8 elements (a 16-byte chunk); the four threads of a
// block agree on its maximum through two lane swaps. Grid: x = rows,
// y = chunks of 256 threads over 16 * KW chunks per row.
template <int FMT>
__global__ __launch_bounds__(256) void quant_blocks_fp8_kernel(
    const bf16_t* __restrict__ src, int64_t K, int64_t ld_src, const int32_t* __restrict__ valid_rows,
    uint8_t* __restrict__ codes, int64_t ld_q, uint8_t* __restrict__ scales, int64_t KW) {
  const int64_t row = blockIdx.x;
  if (valid_rows && row >= (int64_t)*valid_rows) return;
  const int64_t c = (int64_t)blockIdx.y * 256 + threadIdx.x;   // chunk of 8 elements
  if (c >= KW * 16) return;   // a whole group of four threads is in or out
  const int64_t nch = K / 8;
  const uint4 v = c < nch ? *reinterpret_cast<const uint4*>(src + row * ld_src + 8 * c) : make_uint4(0, 0, 0, 0);
  uint32_t m = absmax8(v, 0);
#pragma unroll
  for (int o = 1; o < 4; o <<= 1) {
    const uint32_t t = __shfl_xor(m, o, 64);
    m = t > m ? t : m;
  }
  int e = fp8_scale_exp<FMT>(m, bf2f(m));
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  if (c < nch) *reinterpret_cast<uint2*>(codes + row * ld_q + 8 * c) = to_fp8<FMT>(v, e);
  if ((c & 3) == 0) {
    const int64_t b = c >> 2;   // block
    scales[(((row >> 5) * KW + (b >> 2)) * 32 + (row & 31)) * 4 + (b & 3)] = (uint8_t)(e + 127);
  }
}

// ---- block scales along the token axis, into the transpose (weight gradients)
// src: a token-major [R, C] bf16 matrix whose rows are grouped (group g owns
// rows off[g] .. off[g+1]-1). Column c of group g becomes a run of row c of
// codes_t [C, Rp]: token j of the group at column pos_g + j, with
// pos_g = 128 * (ceil(off[g] / 128) + g), so every group starts on a 128-token
// k-step and the groups never overlap (pos_{g+1} >= pos_g + rows_g + 1).
// Block b of k-step kt (tokens 128 kt + 32 b .. +31 of the group, the last
// one partial) gets e = the per-row rule on that block of the column, clipped
// to [-127, 127]; its byte e + 127 goes to the 32-column interleaved scale
// words of codes_t's rows (word w = pos_g / 128 + kt of row c at
// ((c / 32) * Rp / 128 + w) * 32 + c % 32, byte b). Padding tokens of a
// group's last k-step get code 0 and blocks past the group byte 127; the
// k-steps between groups are not written.
//
// kstep_group_kernel fills tab[q] = the group whose k-steps include padded
// k-step q, or -1: a binary search over the group starts per q.
__global__ __launch_bounds__(256) void kstep_group_kernel(const int32_t* __restrict__ off, int G, int64_t nq,
                                                          int32_t* __restrict__ tab) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= nq) return;
  // the last g with kstart(g) = ceil(off[g] / 128) + g <= q (kstart grows with g)
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)(off[mid] + 127) / 128 + mid <= q) lo = mid;
    else hi = mid - 1;
  }
  const int64_t ks = (int64_t)(off[lo] + 127) / 128 + lo;
  const int64_t rows = off[lo + 1] - off[lo];
  tab[q] = q >= ks && q - ks < (rows + 127) / 128 ? lo : -1;
}

// bounds[0] = lo, bounds[1] = hi: the one-group bounds of a plain matrix
__global__ void set_bounds_kernel(int32_t* __restrict__ bounds, int32_t lo, int32_t hi) {
  if (threadIdx.x == 0) {
    bounds[0] = lo;
    bounds[1] = hi;
  }
}

// Workgroup (x, q): columns CW x .. CW x + CW-1 of padded k-step q (tab[q]'s
// group), CW = 64, or 128 with ROWS. The 128 x CW tile is staged in LDS row
// by row (16-byte chunks); thread t then takes token blocks b of column
// c = t % CW (b = t / CW for CW = 64, 2 (t / 128) and the next for CW = 128):
// each block's maximum, its exponent byte and its 32 codes (two 16-byte
// stores).
// ROWS: the same read also quantizes the tile's rows in 1 x 32 blocks along
// C, exactly as quant_blocks_fp8_kernel does (row codes [R, C] and their
// interleaved scale words, the rows of the group only): a thread's chunks
// share one column chunk, the four lanes of a 32-column block agree on its
// maximum by two lane swaps, and a row's 128 columns are one whole scale
// word (gathered by lane swaps) and one 128-byte line of codes.
template <int FMT, bool ROWS>
__global__ __launch_bounds__(256) void quant_tblocks_fp8_kernel(
    const bf16_t* __restrict__ src, int64_t C, const int32_t* __restrict__ off, const int32_t* __restrict__ tab,
    uint8_t* __restrict__ codes, int64_t Rp, uint8_t* __restrict__ scales, uint8_t* __restrict__ rcodes,
    uint32_t* __restrict__ rscales) {
  constexpr int CW = ROWS ? 128 : 64, NCH = CW / 8, NU = 128 * NCH / 256, NB = CW / 64;
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * CW];
  const int64_t q = blockIdx.y, c0 = (int64_t)blockIdx.x * CW;
  const int g = tab[q];
  if (g < 0) return;
  const int64_t kt = q - ((int64_t)(off[g] + 127) / 128 + g);
  const int64_t t0 = off[g] + 128 * kt;
  const int64_t left = off[g + 1] - t0;
  const int nv = left < 128 ? (int)left : 128;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int ch = tid + 256 * u, r = ch / NCH, cc = ch % NCH;
    const int64_t c = c0 + 8 * cc;
    const uint4 v = r < nv && c < C ? *reinterpret_cast<const uint4*>(src + (t0 + r) * C + c)
                                    : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(tile + r * CW + 8 * cc) = v;
    if constexpr (ROWS) {
      uint32_t m = absmax8(v, 0);
#pragma unroll
      for (int o = 1; o < 4; o <<= 1) {
        const uint32_t t = __shfl_xor(m, o, 64);
        m = t > m ? t : m;
      }
      int e = fp8_scale_exp<FMT>(m, bf2f(m));
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
      // the row's word: blocks 0..3 from the lanes of chunks 0, 4, 8, 12
      const uint32_t by = (uint32_t)(e + 127);
      const uint32_t b1 = (uint32_t)__shfl_xor((int)by, 4, 64), b2 = (uint32_t)__shfl_xor((int)by, 8, 64),
                     b3 = (uint32_t)__shfl_xor((int)by, 12, 64);
      if (r < nv) {
        const int64_t row = t0 + r;
        if (c < C) *reinterpret_cast<uint2*>(rcodes + row * C + c) = to_fp8<FMT>(v, e);
        if (cc == 0) {
          const int64_t KW = (C + 127) / 128;
          rscales[((row >> 5) * KW + (c0 >> 7)) * 32 + (row & 31)] = by | (b1 << 8) | (b2 << 16) | (b3 << 24);
        }
      }
    }
  }
  __syncthreads();
  const int cl = tid % CW;
  const int64_t c = c0 + cl;
  if (c >= C) return;
  const int64_t kw = (int64_t)(off[g] + 127) / 128 + g + kt;   // k-step word of row c
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int b = (tid / CW) * NB + j;
    uint32_t m = 0;
    uint32_t w[16];   // the block's 32 bf16, two to a word, token order
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t lo = tile[(32 * b + 2 * i) * CW + cl], hi = tile[(32 * b + 2 * i + 1) * CW + cl];
      w[i] = lo | (hi << 16);
      m = (lo & 0x7fffu) > m ? (lo & 0x7fffu) : m;
      m = (hi & 0x7fffu) > m ? (hi & 0x7fffu) : m;
    }
    int e = fp8_scale_exp<FMT>(m, bf2f(m));
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    uint2 o[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      o[jj] = to_fp8<FMT>(make_uint4(w[4 * jj], w[4 * jj + 1], w[4 * jj + 2], w[4 * jj + 3]), e);
    uint4* dst = reinterpret_cast<uint4*>(codes + c * Rp + 128 * kw + 32 * b);
    dst[0] = make_uint4(o[0].x, o[0].y, o[1].x, o[1].y);
    dst[1] = make_uint4(o[2].x, o[2].y, o[3].x, o[3].y);
    scales[(((c >> 5) * (Rp / 128) + kw) * 32 + (c & 31)) * 4 + b] = (uint8_t)(e + 127);
  }
}

// ---- per-column quantization into the transpose
// src: G row-major R x C bf16 matrices; codes: G row-major C x R (the
// transposes), so codes row c is src column c quantized like a row above.

constexpr int kTC = 64;                   // columns per workgroup (both passes)

// Pass 1: e[g][c] from max_r |src[g][r][c]|. Thread (rg, cc) covers columns
// c0 + 8cc .. +7 of rows rg, rg + 32, ...; per-column maxima are bit
// patterns, folded over the 32 row groups in LDS.
__global__ __launch_bounds__(256) void col_exp_fp8_kernel(const bf16_t* __restrict__ src, int64_t R,
                                                          int64_t C, int32_t* __restrict__ sexp) {
  const int64_t g = blockIdx.y, c0 = (int64_t)blockIdx.x * kTC;
  const int tid = threadIdx.x, rg = tid >> 3, cc = tid & 7;
  const int64_t c = c0 + 8 * cc;
  const bool cok = c < C;   // C % 8 == 0: a chunk is wholly in or out
  const bf16_t* base = src + g * R * C + (cok ? c : 0);
  uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int64_t r = rg;
  for (; r + 32 * 7 < R; r += 32 * 8) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const uint4*>(base + (r + 32 * u) * C);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w[i] & 0x7fffu, hi = (w[i] >> 16) & 0x7fffu;
        m[2 * i] = lo > m[2 * i] ? lo : m[2 * i];
        m[2 * i + 1] = hi > m[2 * i + 1] ? hi : m[2 * i + 1];
      }
    }
  }
  for (; r < R; r += 32) {
    const uint4 v = *reinterpret_cast<const uint4*>(base + r * C);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = w[i] & 0x7fffu, hi = (w[i] >> 16) & 0x7fffu;
      m[2 * i] = lo > m[2 * i] ? lo : m[2 * i];
      m[2 * i + 1] = hi > m[2 * i + 1] ? hi : m[2 * i + 1];
    }
  }
  __shared__ uint32_t sm[32][kTC + 1];
#pragma unroll
  for (int i = 0; i < 8; ++i) sm[rg][8 * cc + i] = m[i];
  __syncthreads();
  if (tid < kTC && c0 + tid < C) {
    uint32_t mm = 0;
    for (int j = 0; j < 32; ++j) mm = sm[j][tid] > mm ? sm[j][tid] : mm;
    const float amax = bf2f(mm);
    int ex = 0;
    const float mant = frexpf(amax, &ex);
    sexp[g * C + c0 + tid] = mm == 0 ? 0 : (2.0f * mant <= 1.75f ? ex - 9 : ex - 8);
  }
}

// Pass 2: a 64 x 64 block of src (rows r0.., columns c0..) through LDS; thread
// (c, q) writes codes[g][c][r0 + 16q .. +15] as one 16-byte store.
__global__ __launch_bounds__(256) void transpose_quant_fp8_kernel(const bf16_t* __restrict__ src,
                                                                  int64_t R, int64_t C,
                                                                  const int32_t* __restrict__ sexp,
                                                                  uint8_t* __restrict__ codes) {
  const int64_t g = blockIdx.z, r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * kTC;
  const int tid = threadIdx.x;
  __shared__ uint16_t tile[64][kTC + 2];
  // load: row tid >> 2, columns 16 (tid & 3) .. +15 (two 16-byte chunks)
  {
    const int rr = tid >> 2, cq = (tid & 3) * 16;
    const int64_t r = r0 + rr;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t c = c0 + cq + 8 * h;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < R && c < C) v = *reinterpret_cast<const uint4*>(src + (g * R + r) * C + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        tile[rr][cq + 8 * h + 2 * i] = (uint16_t)(w[i] & 0xffffu);
        tile[rr][cq + 8 * h + 2 * i + 1] = (uint16_t)(w[i] >> 16);
      }
    }
  }
  __syncthreads();
  const int cl = tid >> 2, q = tid & 3;
  const int64_t c = c0 + cl, r = r0 + 16 * q;
  if (c >= C || r >= R) return;   // R % 16 == 0: a 16-row piece is wholly in or out
  const int e = sexp[g * C + c];
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = ldexpf(bf2f(tile[16 * q + 4 * i][cl]), -e);
    const float b = ldexpf(bf2f(tile[16 * q + 4 * i + 1][cl]), -e);
    const float cc = ldexpf(bf2f(tile[16 * q + 4 * i + 2][cl]), -e);
    const float d = ldexpf(bf2f(tile[16 * q + 4 * i + 3][cl]), -e);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(cc, d, w, true);
    o[i] = (uint32_t)w;
  }
  *reinterpret_cast<uint4*>(codes + (g * C + c) * R + r) = make_uint4(o[0], o[1], o[2], o[3]);
}

// ---- both orientations with two reads of the source: rows and column
// maxima in one pass, then the transpose with the column exponents.

constexpr int kBR = 64;   // rows per workgroup of the fused pass

__device__ __forceinline__ uint32_t max_pairs(uint32_t a, uint32_t w) {
  // lanes (lo, hi) of two packed 15-bit magnitude pairs
  const uint32_t lo = (a & 0xffffu) > (w & 0x7fffu) ? (a & 0xffffu) : (w & 0x7fffu);
  const uint32_t hi = (a >> 16) > ((w >> 16) & 0x7fffu) ? (a >> 16) : ((w >> 16) & 0x7fffu);
  return lo | (hi << 16);
}

// Workgroup (b, g) quantizes rows 64b .. 64b+63 of src[g] as
// quant_rows_fp8_kernel does, RB rows at a time (TPR = 256 / RB threads per
// row, up to 16 chunks of 8 columns each), and keeps each column's running
// maximum |value|; the RB row slots' maxima are folded in LDS and written as
// partial[g][b][c] (bf16 magnitude bit patterns). C <= 4096 * 8 / RB.
template <int RB>
__global__ __launch_bounds__(256) void rows_colmax_fp8_kernel(const bf16_t* __restrict__ src,
                                                              int64_t R, int64_t C,
                                                              uint8_t* __restrict__ codes,
                                                              int32_t* __restrict__ sexp,
                                                              uint16_t* __restrict__ partial) {
  constexpr int TPR = 256 / RB, NCH = 16;
  const int64_t g = blockIdx.y, b = blockIdx.x, nb = gridDim.x;
  const int tid = threadIdx.x, slot = tid / TPR, t = tid % TPR, wave = tid >> 6;
  const int64_t nch = C / 8;
  __shared__ uint32_t wred[4];
  __shared__ uint16_t scm[32768];
  uint32_t cm[NCH][4];
#pragma unroll
  for (int u = 0; u < NCH; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) cm[u][i] = 0;
  for (int grp = 0; grp < kBR / RB; ++grp) {
    const int64_t row = b * kBR + grp * RB + slot;
    const bool rok = row < R;
    const uint4* s = reinterpret_cast<const uint4*>(src + (g * R + (rok ? row : 0)) * C);
    uint4 cache[NCH];
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int64_t c = t + (int64_t)u * TPR;
      cache[u] = (rok && c < nch) ? s[c] : make_uint4(0, 0, 0, 0);
      m = absmax8(cache[u], m);
    }
    // the row's maximum over its TPR threads
#pragma unroll
    for (int o = (TPR < 64 ? TPR : 64) / 2; o > 0; o >>= 1) {
      const uint32_t x = __shfl_xor(m, o, 64);
      m = x > m ? x : m;
    }
    if constexpr (TPR > 64) {
      if ((tid & 63) == 0) wred[wave] = m;
      __syncthreads();
      m = 0;
#pragma unroll
      for (int w = 0; w < TPR / 64; ++w) {
        const uint32_t x = wred[slot * (TPR / 64) + w];
        m = x > m ? x : m;
      }
      __syncthreads();
    }
    const float amax = bf2f(m);
    int ex = 0;
    const float mant = frexpf(amax, &ex);
    const int e = m == 0 ? 0 : (2.0f * mant <= 1.75f ? ex - 9 : ex - 8);
    if (rok && t == 0) sexp[g * R + row] = e;
    uint2* q = reinterpret_cast<uint2*>(codes + (g * R + row) * C);
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int64_t c = t + (int64_t)u * TPR;
      if (rok && c < nch) q[c] = to_e4m3(cache[u], e);
      cm[u][0] = max_pairs(cm[u][0], cache[u].x);
      cm[u][1] = max_pairs(cm[u][1], cache[u].y);
      cm[u][2] = max_pairs(cm[u][2], cache[u].z);
      cm[u][3] = max_pairs(cm[u][3], cache[u].w);
    }
  }
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int64_t c = t + (int64_t)u * TPR;
    if (c < nch) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        scm[slot * C + c * 8 + 2 * i] = (uint16_t)(cm[u][i] & 0xffffu);
        scm[slot * C + c * 8 + 2 * i + 1] = (uint16_t)(cm[u][i] >> 16);
      }
    }
  }
  __syncthreads();
  for (int64_t col = tid; col < C; col += 256) {
    uint16_t mx = 0;
#pragma unroll
    for (int sl = 0; sl < RB; ++sl) mx = scm[sl * C + col] > mx ? scm[sl * C + col] : mx;
    partial[(g * nb + b) * C + col] = mx;
  }
}

// e[g][c] from the nb partial maxima of column c (eight loaded at a time).
__global__ __launch_bounds__(256) void colmax_reduce_fp8_kernel(const uint16_t* __restrict__ partial,
                                                                int64_t nb, int64_t C,
                                                                int32_t* __restrict__ sexp) {
  const int64_t g = blockIdx.y, col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col >= C) return;
  const uint16_t* p = partial + g * nb * C + col;
  uint32_t mm = 0;
  for (int64_t b0 = 0; b0 < nb; b0 += 8) {
    uint32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = p[(b0 + j < nb ? b0 + j : nb - 1) * C];
#pragma unroll
    for (int j = 0; j < 8; ++j) mm = v[j] > mm ? v[j] : mm;
  }
  const float amax = bf2f(mm);
  int ex = 0;
  const float mant = frexpf(amax, &ex);
  sexp[g * C + col] = mm == 0 ? 0 : (2.0f * mant <= 1.75f ? ex - 9 : ex - 8);
}

// ---- square blocks: one exponent per 32 x 32 square of a weight, both layouts
// G row-major R x C bf16 matrices. Square (i, j) (rows 32i .. 32i+31, columns
// 32j .. 32j+31 of one matrix, partial at its edges) gets e = the per-row rule
// on the square's maximum, clipped to [-127, 127]. A square is a 1 x 32 block
// of every row it covers, in the matrix and in its transpose, so one read
// writes:
//   codes [G*R, C]   and its block-scale words (rows G*R, K = C), and
//   codes_t [G, C, R] and its block-scale words (rows G*C, K = R),
// in moe_quantize_fp8_blocks' 32-row interleaved layout (byte e + 127; blocks
// past the edge hold 127), with the same code in both layouts. A layout whose
// codes pointer is null is skipped.
// Workgroup (x, y, g): the 128 x 128 tile at rows 128y, columns 128x of
// matrix g; wave w takes the tile's rows 32w .. 32w+31 (one row of squares).
// Load i of lane l reads 16 bytes (8 columns) of row 32w + 4i + (l >> 4),
// chunk l & 15, so 16 lanes cover a 256-byte row piece; each lane's 8 chunks
// lie in one square (column block (l & 15) / 4), whose maximum comes from
// lane swaps over the 16 lanes of that square. The codes go to global memory
// (128 bytes per row piece per load) and to LDS; then lane l of wave w reads
// the 4 x 4 byte blocks of columns 4(8w + (l & 7)) .. +3, rows
// 16(l >> 3) .. +15, transposes them and stores 16 codes to each of its 4
// output rows: every store instruction writes eight whole 128-byte lines.
// The scale words of both layouts come from the 16 square exponents in LDS.
constexpr int kSqT = 128;                  // tile edge
constexpr int kSqLd = kSqT + 4;            // LDS row stride in bytes (conflict-free dword reads)

__global__ __launch_bounds__(256) void quant_squares_fp8_kernel(
    const bf16_t* __restrict__ src, int64_t R, int64_t C, uint8_t* __restrict__ codes,
    uint32_t* __restrict__ scales, uint8_t* __restrict__ codes_t, uint32_t* __restrict__ scales_t) {
  __shared__ __attribute__((aligned(16))) uint8_t q_s[kSqT * kSqLd];
  __shared__ uint32_t e_s[4][4];               // byte e + 127 of square (row block, column block)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t g = blockIdx.z, r0 = (int64_t)blockIdx.y * kSqT, c0 = (int64_t)blockIdx.x * kSqT;
  const bf16_t* x = src + g * R * C;
  // phase 1 (C % 8 == 0: an 8-column chunk is inside or outside whole)
  const int ch = lane & 15, rl = lane >> 4;
  const int64_t col = c0 + 8 * ch;
  uint4 v[8];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = r0 + 32 * wave + 4 * i + rl;
    v[i] = row < R && col < C ? *reinterpret_cast<const uint4*>(x + row * C + col) : make_uint4(0, 0, 0, 0);
    m = absmax8(v[i], m);
  }
  // the square's 16 lanes: lane bits 0, 1 (its 4 chunks) and 4, 5 (row groups)
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    if (o == 4 || o == 8) continue;
    const uint32_t t = __shfl_xor(m, o, 64);
    m = t > m ? t : m;
  }
  int e = fp8_scale_exp<0>(m, bf2f(m));
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  if ((lane & 0x33) == 0) e_s[wave][ch >> 2] = (uint32_t)(e + 127);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rloc = 32 * wave + 4 * i + rl;
    const int64_t row = r0 + rloc;
    const uint2 q = to_fp8<0>(v[i], e);
    if (codes && row < R && col < C) *reinterpret_cast<uint2*>(codes + (g * R + row) * C + col) = q;
    *reinterpret_cast<uint32_t*>(q_s + rloc * kSqLd + 8 * ch) = q.x;
    *reinterpret_cast<uint32_t*>(q_s + rloc * kSqLd + 8 * ch + 4) = q.y;
  }
  __syncthreads();
  // the rows' scale words: tile row t takes the four column blocks' bytes of
  // its row block
  if (codes && tid < kSqT && r0 + tid < R) {
    const int rb = tid >> 5;
    const int64_t rowg = g * R + r0 + tid, KW = (C + kSqT - 1) / kSqT;
    scales[((rowg >> 5) * KW + c0 / kSqT) * 32 + (rowg & 31)] =
        e_s[rb][0] | (e_s[rb][1] << 8) | (e_s[rb][2] << 16) | (e_s[rb][3] << 24);
  }
  if (!codes_t) return;
  // phase 2: output rows (tile columns) 4cq .. 4cq+3, k (tile rows) 16rq .. 16rq+15
  const int cq = 8 * wave + (lane & 7), rq = lane >> 3;
  uint32_t o[4][4];   // o[c][i]: output row 4cq + c, k 16rq + 4i .. +3
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
      w[s2] = *reinterpret_cast<const uint32_t*>(q_s + (16 * rq + 4 * i + s2) * kSqLd + 4 * cq);
    // 4 x 4 byte transpose: byte c of rows 0..3 -> bytes 0..3 of o[c][i]
#pragma unroll
    for (int c = 0; c < 4; ++c)
      o[c][i] = ((w[0] >> (8 * c)) & 0xffu) | (((w[1] >> (8 * c)) & 0xffu) << 8) |
                (((w[2] >> (8 * c)) & 0xffu) << 16) | (((w[3] >> (8 * c)) & 0xffu) << 24);
  }
  const int64_t k0 = r0 + 16 * rq;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t col = c0 + 4 * cq + c;
    if (col < C && k0 < R)
      *reinterpret_cast<uint4*>(codes_t + (g * C + col) * R + k0) = make_uint4(o[c][0], o[c][1], o[c][2], o[c][3]);
  }
  // transposed scale words: output row c0 + t takes the four row blocks' bytes
  // of its column block
  if (tid < kSqT && c0 + tid < C) {
    const int cb = tid >> 5;
    const int64_t rowt = g * C + c0 + tid, KWt = (R + kSqT - 1) / kSqT;
    scales_t[((rowt >> 5) * KWt + r0 / kSqT) * 32 + (rowt & 31)] =
        e_s[0][cb] | (e_s[1][cb] << 8) | (e_s[2][cb] << 16) | (e_s[3][cb] << 24);
  }
}

}  // namespace

size_t quant_fp8_both_ws(int64_t G, int64_t R, int64_t C) {
  return ((size_t)G * ((R + kBR - 1) / kBR) * C * 2 + 255) / 256 * 256;
}

// Rows [G*R, C] and transposes [G, C, R] of G row-major R x C matrices; ws
// holds quant_fp8_both_ws bytes of partial column maxima. C % 16 == 0,
// C <= 32768, R % 16 == 0.
hipError_t launch_quant_fp8_both(const void* src, int64_t G, int64_t R, int64_t C, void* codes,
                                 int32_t* sexp, void* codes_t, int32_t* sexp_t, void* ws,
                                 hipStream_t st) {
  if (G == 0 || R == 0 || C == 0) return hipSuccess;
  const dim3 grid((unsigned)((R + kBR - 1) / kBR), (unsigned)G);
  const bf16_t* x = (const bf16_t*)src;
  uint16_t* part = (uint16_t*)ws;
  if (C <= 4096)
    hipLaunchKernelGGL(rows_colmax_fp8_kernel<8>, grid, dim3(256), 0, st, x, R, C, (uint8_t*)codes, sexp, part);
  else if (C <= 8192)
    hipLaunchKernelGGL(rows_colmax_fp8_kernel<4>, grid, dim3(256), 0, st, x, R, C, (uint8_t*)codes, sexp, part);
  else if (C <= 16384)
    hipLaunchKernelGGL(rows_colmax_fp8_kernel<2>, grid, dim3(256), 0, st, x, R, C, (uint8_t*)codes, sexp, part);
  else if (C <= 32768)
    hipLaunchKernelGGL(rows_colmax_fp8_kernel<1>, grid, dim3(256), 0, st, x, R, C, (uint8_t*)codes, sexp, part);
  else
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(colmax_reduce_fp8_kernel, dim3((unsigned)((C + 255) / 256), (unsigned)G),
                     dim3(256), 0, st, (const uint16_t*)part, (int64_t)grid.x, C, sexp_t);
  const unsigned nc = (unsigned)((C + kTC - 1) / kTC);
  hipLaunchKernelGGL(transpose_quant_fp8_kernel, dim3(nc, (unsigned)((R + 63) / 64), (unsigned)G),
                     dim3(256), 0, st, x, R, C, (const int32_t*)sexp_t, (uint8_t*)codes_t);
  return hipGetLastError();
}

hipError_t launch_quant_fp8_t(const void* src, int64_t G, int64_t R, int64_t C, void* codes,
                              int32_t* sexp, hipStream_t st) {
  if (G == 0 || R == 0 || C == 0) return hipSuccess;
  const unsigned nc = (unsigned)((C + kTC - 1) / kTC);
  hipLaunchKernelGGL(col_exp_fp8_kernel, dim3(nc, (unsigned)G), dim3(256), 0, st,
                     (const bf16_t*)src, R, C, sexp);
  hipLaunchKernelGGL(transpose_quant_fp8_kernel, dim3(nc, (unsigned)((R + 63) / 64), (unsigned)G),
                     dim3(256), 0, st, (const bf16_t*)src, R, C, (const int32_t*)sexp,
                     (uint8_t*)codes);
  return hipGetLastError();
}

// fmt: 0 = E4M3, 1 = E5M2
hipError_t launch_quant_fp8(const void* src, int64_t rows, int64_t K, int64_t ld_src,
                            const int32_t* valid_rows, void* codes, int64_t ld_q, int32_t* sexp,
                            hipStream_t st, int fmt) {
  if (rows == 0) return hipSuccess;
  if (fmt == 1)
    hipLaunchKernelGGL(quant_rows_fp8_kernel<1>, dim3((unsigned)rows), dim3(kQThreads), 0, st,
                       (const bf16_t*)src, K, ld_src, valid_rows, (uint8_t*)codes, ld_q, sexp);
  else
    hipLaunchKernelGGL(quant_rows_fp8_kernel<0>, dim3((unsigned)rows), dim3(kQThreads), 0, st,
                       (const bf16_t*)src, K, ld_src, valid_rows, (uint8_t*)codes, ld_q, sexp);
  return hipGetLastError();
}

// Token-axis block quantization of a grouped token-major [R, C] matrix into
// its transpose (see quant_tblocks_fp8_kernel). off: G + 1 group bounds on the
// device; tab: nq = Rp / 128 ints of scratch; Rp = 128 * (ceil(R / 128) + G).
// rcodes / rscales (both or neither): also the rows' 1 x 32 block
// quantization of src (codes [R, C], row stride C, and 32-row interleaved
// scale bytes), the rows of the groups only. C % 8 == 0.
hipError_t launch_quant_fp8_tblocks(const void* src, int64_t R, int64_t C, const int32_t* off, int G,
                                    int32_t* tab, void* codes_t, uint8_t* scales, hipStream_t st, int fmt,
                                    void* rcodes, uint8_t* rscales) {
  const int64_t Rp = 128 * ((R + 127) / 128 + G), nq = Rp / 128;
  if (R == 0 || C == 0) return hipSuccess;
  hipLaunchKernelGGL(kstep_group_kernel, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, st, off, G, nq, tab);
  const bool rows = rcodes != nullptr;
  const int64_t cw = rows ? 128 : 64;   // the kernel's tile width
  const dim3 grid((unsigned)((C + cw - 1) / cw), (unsigned)nq);
  const bf16_t* x = (const bf16_t*)src;
  uint8_t* ct = (uint8_t*)codes_t;
  uint8_t* rc = (uint8_t*)rcodes;
  uint32_t* rs = (uint32_t*)rscales;
  if (fmt == 1 && rows)
    hipLaunchKernelGGL((quant_tblocks_fp8_kernel<1, true>), grid, dim3(256), 0, st, x, C, off, tab, ct, Rp, scales,
                       rc, rs);
  else if (fmt == 1)
    hipLaunchKernelGGL((quant_tblocks_fp8_kernel<1, false>), grid, dim3(256), 0, st, x, C, off, tab, ct, Rp, scales,
                       rc, rs);
  else if (rows)
    hipLaunchKernelGGL((quant_tblocks_fp8_kernel<0, true>), grid, dim3(256), 0, st, x, C, off, tab, ct, Rp, scales,
                       rc, rs);
  else
    hipLaunchKernelGGL((quant_tblocks_fp8_kernel<0, false>), grid, dim3(256), 0, st, x, C, off, tab, ct, Rp, scales,
                       rc, rs);
  return hipGetLastError();
}

hipError_t launch_set_bounds(int32_t* bounds, int32_t lo, int32_t hi, hipStream_t st) {
  hipLaunchKernelGGL(set_bounds_kernel, dim3(1), dim3(64), 0, st, bounds, lo, hi);
  return hipGetLastError();
}

// Block-scaled rows: codes [rows, K] (row stride ld_q) and 32-row
// interleaved scale words (ceil(rows / 32) * 32 * ceil(K / 128) words).
// K % 8 == 0, 16-byte aligned source rows.
// fmt: 0 = E4M3, 1 = E5M2.
hipError_t launch_quant_fp8_blocks(const void* src, int64_t rows, int64_t K, int64_t ld_src,
                                   const int32_t* valid_rows, void* codes, int64_t ld_q,
                                   uint8_t* scales, hipStream_t st, int fmt) {
  if (rows == 0 || K == 0) return hipSuccess;
  const int64_t KW = (K + 127) / 128;
  const dim3 grid((unsigned)rows, (unsigned)((KW * 16 + 255) / 256));
  if (fmt == 1)
    hipLaunchKernelGGL(quant_blocks_fp8_kernel<1>, grid, dim3(256), 0, st, (const bf16_t*)src, K, ld_src,
                       valid_rows, (uint8_t*)codes, ld_q, scales, KW);
  else
    hipLaunchKernelGGL(quant_blocks_fp8_kernel<0>, grid, dim3(256), 0, st, (const bf16_t*)src, K, ld_src,
                       valid_rows, (uint8_t*)codes, ld_q, scales, KW);
  return hipGetLastError();
}

// Square-block weights, both layouts (quant_squares_fp8_kernel; codes or
// codes_t null: that layout is skipped). R % 16 == 0, C % 16 == 0; scales:
// ceil(G*R / 32) * 32 * ceil(C / 128) words, scales_t: ceil(G*C / 32) * 32 *
// ceil(R / 128) words.
hipError_t launch_quant_fp8_squares(const void* src, int64_t G, int64_t R, int64_t C, void* codes,
                                    uint8_t* scales, void* codes_t, uint8_t* scales_t, hipStream_t st) {
  if (G == 0 || R == 0 || C == 0) return hipSuccess;
  const dim3 grid((unsigned)((C + kSqT - 1) / kSqT), (unsigned)((R + kSqT - 1) / kSqT), (unsigned)G);
  hipLaunchKernelGGL(quant_squares_fp8_kernel, grid, dim3(256), 0, st, (const bf16_t*)src, R, C,
                     (uint8_t*)codes, (uint32_t*)scales, (uint8_t*)codes_t, (uint32_t*)scales_t);
  return hipGetLastError();
}

}  // namespace moe
