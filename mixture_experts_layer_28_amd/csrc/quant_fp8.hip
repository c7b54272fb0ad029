// Per-row FP8 (OCP E4M3) quantization with power-of-two scales, the input
// side of the FP8 forward GEMMs. Row i of a bf16 matrix becomes
//   codes[i][k] = E4M3 nearest (ties to even) of x[i][k] * 2^-e_i,
// e_i = the smallest integer with max_k |x[i][k]| <= 448 * 2^e_i (0 for an
// all-zero row). Multiplying by a power of two is exact, so the conversion
// instruction's rounding is the only rounding; the codes are a bit-exact
// function of the input. Inputs must be finite.
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

__device__ __forceinline__ uint32_t absmax8(uint4 v, uint32_t m) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // |bf16| bit patterns order like their magnitudes (finite inputs)
    const uint32_t lo = w[i] & 0x7fffu, hi = (w[i] >> 16) & 0x7fffu;
    m = lo > m ? lo : m;
    m = hi > m ? hi : m;
  }
  return m;
}

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
  const float amax = bf2f(m);
  int ex = 0;
  const float mant = frexpf(amax, &ex);
  const int e = m == 0 ? 0 : (2.0f * mant <= 1.75f ? ex - 9 : ex - 8);
  if (tid == 0) sexp[row] = e;
#pragma unroll
  for (int u = 0; u < kQCache; ++u) {
    const int64_t c = tid + (int64_t)u * kQThreads;
    if (c < nch) q[c] = to_e4m3(cache[u], e);
  }
  for (int64_t c = tid + (int64_t)kQCache * kQThreads; c < nch; c += kQThreads) q[c] = to_e4m3(s[c], e);
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

hipError_t launch_quant_fp8(const void* src, int64_t rows, int64_t K, int64_t ld_src,
                            const int32_t* valid_rows, void* codes, int64_t ld_q, int32_t* sexp,
                            hipStream_t st) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_fp8_kernel, dim3((unsigned)rows), dim3(kQThreads), 0, st,
                     (const bf16_t*)src, K, ld_src, valid_rows, (uint8_t*)codes, ld_q, sexp);
  return hipGetLastError();
}

}  // namespace moe
