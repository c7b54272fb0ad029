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

}  // namespace

hipError_t launch_quant_fp8(const void* src, int64_t rows, int64_t K, int64_t ld_src,
                            const int32_t* valid_rows, void* codes, int64_t ld_q, int32_t* sexp,
                            hipStream_t st) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_fp8_kernel, dim3((unsigned)rows), dim3(kQThreads), 0, st,
                     (const bf16_t*)src, K, ld_src, valid_rows, (uint8_t*)codes, ld_q, sexp);
  return hipGetLastError();
}

}  // namespace moe
