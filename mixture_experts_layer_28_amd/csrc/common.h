// Device helpers shared by the libmoe kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bfloat16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> a packed bfloat16 pair (lo in bits 0-15), round to nearest
// even, NaN stays NaN: gfx950's v_cvt_pk_bf16_f32, one instruction per pair.
// On every non-NaN float32 input it gives the same bits as integer
// round-to-nearest-even (u + 0x7fff + ((u >> 16) & 1)) >> 16 (checked over
// all 2^32 inputs on the device); an integer version compiles to a
// branch per element for the NaN case.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// float -> bfloat16 bits, same rounding
__device__ __forceinline__ uint32_t f2bf(float f) { return pack_bf2(f, 0.0f) & 0xffffu; }

// 8 consecutive elements <-> 8 floats, for either storage type
template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* v) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    v[0] = bf2f(u.x & 0xffff); v[1] = bf2f(u.x >> 16);
    v[2] = bf2f(u.y & 0xffff); v[3] = bf2f(u.y >> 16);
    v[4] = bf2f(u.z & 0xffff); v[5] = bf2f(u.z >> 16);
    v[6] = bf2f(u.w & 0xffff); v[7] = bf2f(u.w >> 16);
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* v) {
    uint4 u;
    u.x = pack_bf2(v[0], v[1]); u.y = pack_bf2(v[2], v[3]);
    u.z = pack_bf2(v[4], v[5]); u.w = pack_bf2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = u;
  }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* v) {
    float4 a = reinterpret_cast<const float4*>(p)[0];
    float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// ------------------------------------------------------------ FP8 codes
// Largest |bf16| bit pattern of eight packed bf16 and m (finite inputs:
// the patterns order like the magnitudes).
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

// FP8 formats: 0 = OCP E4M3 (largest magnitude 1.75 * 2^8), 1 = OCP E5M2
// (1.75 * 2^15). The scale rule of a maximum amax = mant * 2^ex (mant in
// [0.5, 1)): the smallest e with amax <= 1.75 * 2^(B + e).
template <int FMT>
__device__ __forceinline__ int fp8_scale_exp(uint32_t m_bits, float amax) {
  constexpr int B = FMT == 1 ? 15 : 8;
  int ex = 0;
  const float mant = frexpf(amax, &ex);
  return m_bits == 0 ? 0 : (2.0f * mant <= 1.75f ? ex - 1 - B : ex - B);
}

// eight bf16 scaled by 2^-e -> eight FP8 codes (byte i = element i), E4M3 or
// E5M2 (round to nearest even either way)
template <int FMT = 0>
__device__ __forceinline__ uint2 to_fp8(uint4 v, int e) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float a = ldexpf(bf2f(w[2 * h] & 0xffffu), -e);
    const float b = ldexpf(bf2f(w[2 * h] >> 16), -e);
    const float c = ldexpf(bf2f(w[2 * h + 1] & 0xffffu), -e);
    const float d = ldexpf(bf2f(w[2 * h + 1] >> 16), -e);
    int r;
    if constexpr (FMT == 1) {
      r = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
      r = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, r, true);
    } else {
      r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
      r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    }
    o[h] = (uint32_t)r;
  }
  return make_uint2(o[0], o[1]);
}

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16_t v) { return bf2f(v); }

// ------------------------------------------------------------ activations
// logistic function from the hardware exp2 and reciprocal (a few ulp in
// float32; used by the GEMM epilogues, whose outputs are rounded to bf16 or
// compared at 1e-5). Saturates cleanly: a -> -inf gives 1/inf = 0.
__device__ __forceinline__ float sigmoidf_(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * -1.4426950408889634f));
}
__device__ __forceinline__ float silu_f(float a) { return a * sigmoidf_(a); }
__device__ __forceinline__ float dsilu_f(float a) {
  float s = sigmoidf_(a);
  return s * (1.0f + a * (1.0f - s));
}
// exact (erf) GELU and its derivative
// erf by the rational approximation of Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (after Hastings):
//   erf(x) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),
//   t = 1 / (1 + p x), x >= 0, odd extension for x < 0,
// |error| <= 1.5e-7 in exact arithmetic, 5.3e-7 as evaluated here in float32.
// Branch-free: the library erff takes a branch per range, which made the
// GELU epilogues diverge per element. e = exp(-x^2) is passed in so the
// GELU derivative can share it with the normal density.
__device__ __forceinline__ float erf_as(float x, float e) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  const float poly =
      t * (0.254829592f +
           t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  return copysignf(1.0f - poly * e, x);
}
// exp(-a^2 / 2), the Gaussian factor of GELU's CDF and density at a
__device__ __forceinline__ float gauss_f(float a) {
  return __builtin_amdgcn_exp2f(a * a * -0.72134752044448170f);   // -log2(e) / 2
}
// GELU with the exact normal CDF: a * Phi(a), Phi(a) = (1 + erf(a / sqrt 2)) / 2
__device__ __forceinline__ float gelu_f(float a) {
  return 0.5f * a * (1.0f + erf_as(a * 0.70710678118654752f, gauss_f(a)));
}
// d gelu / da = Phi(a) + a phi(a), phi(a) = exp(-a^2 / 2) / sqrt(2 pi)
__device__ __forceinline__ float dgelu_f(float a) {
  const float e = gauss_f(a);
  const float cdf = 0.5f * (1.0f + erf_as(a * 0.70710678118654752f, e));
  return cdf + a * (e * 0.39894228040143268f);
}

// ------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// ------------------------------------------------------------ GEMM plumbing
// Epilogue kinds of the grouped GEMMs (applied to float32 accumulators).
enum Epi : int {
  EPI_STORE = 0,       // C = acc (+ col_bias)
  EPI_SWIGLU_FWD = 1,  // fused gate/up tile: C = H = silu(a) * b, aux = [a | b]
  EPI_GELU_FWD = 2,    // C = H = gelu(acc), aux = a = acc
  EPI_SWIGLU_BWD = 3,  // acc = dH; reads aux = [a | b]; C = [da | db]
  EPI_GELU_BWD = 4,    // acc = dH; reads aux = a; C = da
  EPI_STORE_F32 = 5,   // bf16 GEMM with a float32 C = acc (router partial products)
};

// How the groups (experts) of one grouped GEMM are shaped.
enum Rag : int {
  RAG_M = 0,       // group g has M_g = off[g+1]-off[g] rows (forward, dgrad)
  RAG_K = 1,       // group g has K_g = off[g+1]-off[g] (wgrad: reduce over the expert's rows)
  RAG_NONE = 2,    // G groups of identical M x N x K; group g's first row is g*M (or g*K)
};

// One operand of a grouped GEMM. Element (i, kk) of A (i = row of C) lives at
// base + i*ld + kk when kmajor, else base + kk*ld + i; likewise for B with
// i = column of C. Per group the base moves by r0*ld ("row-indexed": the
// operand is a routed-row tensor whose rows start at the group's first row
// r0) or by g*gstride (a stacked per-expert weight).
struct Operand {
  const void* base;
  int64_t ld;
  int64_t gstride;
  int rowidx;
};

struct GemmArgs {
  Operand a, b;
  void* c; int64_t ldc; int64_t c_gstride; int c_rowidx;
  void* aux; int64_t ldaux; int64_t aux_gstride; int aux_rowidx;  // epilogue side tensor
  const int32_t* offsets;   // [G+1] device (RAG_M / RAG_K)
  int G;
  int64_t M, N, K;          // the non-ragged sizes; for EPI_SWIGLU_FWD N = f (H columns)
  int64_t fdim;             // f (column split of [a | b]) for the SwiGLU epilogues
  const float* col_bias;    // EPI_STORE: added per output column, or null
  int64_t max_rows;         // RAG_M: upper bound of sum of M_g (grid sizing)
  int k_splits;             // split-K partitions (fp32 GEMM, RAG_NONE only); 1 = none
  // FP8 GEMM: power-of-two scale exponents, per A row (indexed like A's rows)
  // and per weight row (group g at b_sexp + g * b_sexp_gstride). With
  // blk_scales, both point at block scales instead: one 8-bit exponent byte
  // (e + 127) per 32 elements along K, four to a 32-bit word per 128-k step,
  // words 32-row interleaved (word w of matrix row r at (r / 32 * ceil(K /
  // 128) + w) * 32 + r % 32); A's rows are indexed like A's, group g's weight
  // rows start at matrix row g * b_sexp_gstride.
  const int32_t* a_sexp;
  const int32_t* b_sexp;
  int64_t b_sexp_gstride;
  int blk_scales;
  // bf16 RAG_M plain-store GEMMs: split-K of each XCD's last, partial round of
  // tiles. tail_ws (null = off) holds tail_counters(cus) zeroed int32 counters,
  // then the fp32 partial accumulators; tail_cus = CUs per XCD.
  void* tail_ws;
  int tail_cus;
};

// Tail split-K workspace (see GemmArgs::tail_ws) for `cus` CUs per XCD: a
// counter per possible tail tile (at most cus/2 per XCD), then a 256 KiB
// partial per split item (at most cus per XCD).
__host__ __device__ inline size_t tail_counter_bytes(int cus) { return ((size_t)8 * cus * 4 + 255) / 256 * 256; }
__host__ __device__ inline size_t tail_ws_bytes(int cus) { return tail_counter_bytes(cus) + (size_t)8 * cus * 262144; }

}  // namespace moe
