// Router top-k, load-balance statistics, permute (local dispatch), combine,
// and their backward companions. All HBM-bound or latency-bound; each is a
// plain streaming kernel with 16-byte accesses and fixed reduction orders.
#include "gemm_tile.h"

namespace moe {

typedef uint32_t v4u32_ __attribute__((ext_vector_type(4)));

// --------------------------------------------------------------- router
// One wave per token. Experts e = lane + 64*i live in registers (EPL per lane).
// Softmax is max-subtracted; top-k is k rounds of a wave arg-max on the
// selection key with ties to the lower expert index.
// noisy-gate noise from a uniform draw, evaluated in float64
__device__ __forceinline__ float gumbel_g(float u) {
  return (float)(-log(-log((double)u + 1e-10) + 1e-10));
}

template <int EPL>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits, int T,
                                                          int E, int k, int score,
                                                          const float* __restrict__ sel_bias,
                                                          int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ gate,
                                                          float* __restrict__ scores,
                                                          float* __restrict__ lse,
                                                          const float* __restrict__ gumbel_u,
                                                          float tau) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* lrow = logits + t * E;
  float s[EPL], key[EPL], l[EPL], m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    l[i] = e < E ? lrow[e] : -INFINITY;
    if (gumbel_u && e < E) l[i] = (l[i] + gumbel_g(gumbel_u[t * E + e])) / tau;
    m = fmaxf(m, l[i]);
  }
  m = wave_max(m);
  float ex[EPL], sum = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    ex[i] = e < E ? expf(l[i] - m) : 0.f;
    sum += ex[i];
  }
  sum = wave_sum(sum);
  if (lse && lane == 0) lse[t] = m + logf(sum);
  if (score == 0) {
    const float inv = 1.0f / sum;
#pragma unroll
    for (int i = 0; i < EPL; ++i) s[i] = ex[i] * inv;
  } else {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      s[i] = e < E ? 1.0f / (1.0f + expf(-l[i])) : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      scores[t * E + e] = s[i];
      key[i] = s[i] + (sel_bias ? sel_bias[e] : 0.f);
    } else {
      key[i] = -INFINITY;
    }
  }
  float chosen_sum = 0.f;
  float my_s = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bk = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (key[i] > bk) { bk = key[i]; be = lane + 64 * i; }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ok = __shfl_xor(bk, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ok > bk || (ok == bk && oe < be)) { bk = ok; be = oe; }
    }
    const int owner = be & 63, slot = be >> 6;
    float sv = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (i == slot) {
        sv = s[i];
        if (lane == owner) key[i] = -INFINITY;
      }
    sv = __shfl(sv, owner, 64);
    chosen_sum += sv;
    if (lane == j) { my_s = sv; my_e = be; }
  }
  if (lane < k) {
    topk_idx[t * k + lane] = my_e;
    gate[t * k + lane] = my_s / chosen_sum;
  }
}

hipError_t launch_router_topk(const float* logits, int T, int E, int k, int score,
                              const float* sel_bias, int32_t* topk, float* gate, float* scores,
                              float* lse, const float* gumbel_u, float tau, hipStream_t st) {
  dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(router_topk_kernel<1>, grid, block, 0, st, logits, T, E, k, score, sel_bias, topk, gate, scores, lse, gumbel_u, tau);
  else if (E <= 128)
    hipLaunchKernelGGL(router_topk_kernel<2>, grid, block, 0, st, logits, T, E, k, score, sel_bias, topk, gate, scores, lse, gumbel_u, tau);
  else if (E <= 256)
    hipLaunchKernelGGL(router_topk_kernel<4>, grid, block, 0, st, logits, T, E, k, score, sel_bias, topk, gate, scores, lse, gumbel_u, tau);
  else
    hipLaunchKernelGGL(router_topk_kernel<16>, grid, block, 0, st, logits, T, E, k, score, sel_bias, topk, gate, scores, lse, gumbel_u, tau);
  return hipGetLastError();
}

// Fused router for few experts (E <= EMAX = 8): logits, scores and top-k in one
// pass. A wave owns TPW tokens; lane l covers columns 8*(l + 64*q); the
// per-lane partial dot products are summed across the wave (butterfly), then
// every lane holds all E logits of its tokens and lanes 0..TPW-1 finish one
// token each. x is read once from HBM; W_r rows are re-read from cache.
template <typename TX, int EMAX, int TPW>
__global__ __launch_bounds__(256) void router_small_kernel(
    const TX* __restrict__ x, const float* __restrict__ w_r, const float* __restrict__ logit_bias,
    const float* __restrict__ sel_bias, int T, int E, int64_t d, int k, int score,
    int32_t* __restrict__ topk_idx, float* __restrict__ gate, float* __restrict__ scores,
    float* __restrict__ lse, const float* __restrict__ gumbel_u, float tau) {
  const int lane = threadIdx.x & 63;
  const int64_t t0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW;
  if (t0 >= T) return;
  float acc[TPW][EMAX];
#pragma unroll
  for (int a = 0; a < TPW; ++a)
#pragma unroll
    for (int e = 0; e < EMAX; ++e) acc[a][e] = 0.f;
  for (int64_t c = lane * 8; c < d; c += 512) {
    float xv[TPW][8];
#pragma unroll
    for (int a = 0; a < TPW; ++a) {
      const int64_t t = t0 + a < T ? t0 + a : T - 1;
      Vec8<TX>::load(x + t * d + c, xv[a]);
    }
    // every expert row is loaded without a branch (rows e >= E repeat row 0;
    // their sums are never used), so the loads of an iteration stay in flight
    // together instead of each waiting behind its own branch
    float wv[EMAX][8];
#pragma unroll
    for (int e = 0; e < EMAX; ++e) Vec8<float>::load(w_r + (int64_t)(e < E ? e : 0) * d + c, wv[e]);
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
#pragma unroll
      for (int a = 0; a < TPW; ++a)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[a][e] = fmaf(xv[a][i], wv[e][i], acc[a][e]);
  }
#pragma unroll
  for (int a = 0; a < TPW; ++a)
#pragma unroll
    for (int e = 0; e < EMAX; ++e) acc[a][e] = wave_sum(acc[a][e]);
  // lane a < TPW finishes token t0 + a (a select chain keeps acc in registers)
  float l[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    float v = acc[0][e];
#pragma unroll
    for (int a = 1; a < TPW; ++a) v = lane == a ? acc[a][e] : v;
    l[e] = v;
  }
  const int64_t t = t0 + lane;
  if (lane >= TPW || t >= T) return;
  float sc[EMAX], key[EMAX], ex[EMAX];
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < E) {
      l[e] += logit_bias ? logit_bias[e] : 0.f;
      if (gumbel_u) l[e] = (l[e] + gumbel_g(gumbel_u[(int64_t)t * E + e])) / tau;
      m = fmaxf(m, l[e]);
    }
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    ex[e] = e < E ? expf(l[e] - m) : 0.f;
    sum += ex[e];
  }
  if (lse) lse[t] = m + logf(sum);
  if (score == 0) {
    const float inv = 1.0f / sum;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) sc[e] = ex[e] * inv;
  } else {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) sc[e] = e < E ? 1.0f / (1.0f + expf(-l[e])) : 0.f;
  }
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    if (e < E) scores[t * E + e] = sc[e];
    key[e] = e < E ? sc[e] + (sel_bias ? sel_bias[e] : 0.f) : -INFINITY;
  }
  float chosen = 0.f;
  for (int j = 0; j < k; ++j) {
    float bk = -INFINITY;
    int be = 0;
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (key[e] > bk) { bk = key[e]; be = e; }
    float sv = 0.f;
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (e == be) { sv = sc[e]; key[e] = -INFINITY; }
    topk_idx[t * k + j] = be;
    gate[t * k + j] = sv;
    chosen += sv;
  }
  const float inv = 1.0f / chosen;
  for (int j = 0; j < k; ++j) gate[t * k + j] *= inv;
}

hipError_t launch_router_small(const void* x, bool bf16, const float* w_r, const float* logit_bias,
                               const float* sel_bias, int T, int E, int64_t d, int k, int score,
                               int32_t* topk, float* gate, float* scores, float* lse,
                               const float* gumbel_u, float tau, hipStream_t st) {
  constexpr int TPW = 8;
  const dim3 grid((unsigned)((T + 4 * TPW - 1) / (4 * TPW))), block(256);
  if (bf16)
    hipLaunchKernelGGL((router_small_kernel<bf16_t, 8, TPW>), grid, block, 0, st,
                       (const bf16_t*)x, w_r, logit_bias, sel_bias, T, E, d, k, score, topk, gate,
                       scores, lse, gumbel_u, tau);
  else
    hipLaunchKernelGGL((router_small_kernel<float, 8, TPW>), grid, block, 0, st,
                       (const float*)x, w_r, logit_bias, sel_bias, T, E, d, k, score, topk, gate,
                       scores, lse, gumbel_u, tau);
  return hipGetLastError();
}

// ------------------------------------------------------------ aux stats
// Pass 1: block b covers tokens [256b, 256b+256). Per expert, the scores
// are summed in float64 by G = 256 / min(E, 256) interleaved token groups
// (group g takes tokens t0+g, t0+g+G, ...) whose partials are then added in
// group order; assignments are counted in an LDS histogram and the squared
// lse values summed by a fixed-shape tree. Every order is fixed, so the
// result does not change from run to run.
__global__ __launch_bounds__(256) void aux_partial_kernel(const float* __restrict__ scores,
                                                          const int32_t* __restrict__ topk,
                                                          const float* __restrict__ lse, int T,
                                                          int E, int k, double* __restrict__ pz,
                                                          int32_t* __restrict__ pc,
                                                          double* __restrict__ pl) {
  __shared__ int hist[1024];
  __shared__ double part[256];
  __shared__ double wl[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int t0 = b * 256, t1 = min(T, t0 + 256);
  for (int i = t0 * k + tid; i < t1 * k; i += 256) atomicAdd(&hist[topk[i]], 1);

  const int W = min(E, 256), G = 256 / W;
  for (int e0 = 0; e0 < E; e0 += W) {
    const int e = e0 + tid % W, g = tid / W;
    double z = 0.0;
    if (g < G && e < E) {
#pragma unroll 8
      for (int t = t0 + g; t < t1; t += G) z += (double)scores[(int64_t)t * E + e];
    }
    part[tid] = z;
    __syncthreads();
    if (tid < W && e0 + tid < E) {
      double s = 0.0;
      for (int j = 0; j < G; ++j) s += part[j * W + tid];
      pz[(int64_t)b * E + e0 + tid] = s;
    }
    __syncthreads();
  }
  for (int e = tid; e < E; e += 256) pc[(int64_t)b * E + e] = hist[e];

  double zl = 0.0;
  if (lse && t0 + tid < t1) {
    const double v = (double)lse[t0 + tid];
    zl = v * v;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) zl += __shfl_xor(zl, o, 64);
  if ((tid & 63) == 0) wl[tid >> 6] = zl;
  __syncthreads();
  if (tid == 0) pl[b] = ((wl[0] + wl[1]) + wl[2]) + wl[3];
}

// Pass 2 (one block): fold the partials in block order.
__global__ __launch_bounds__(256) void aux_final_kernel(const double* __restrict__ pz,
                                                        const int32_t* __restrict__ pc,
                                                        const double* __restrict__ pl, int nb,
                                                        int T, int E, int k,
                                                        int32_t* __restrict__ counts,
                                                        float* __restrict__ y,
                                                        float* __restrict__ z,
                                                        float* __restrict__ out3) {
  __shared__ double red[256];
  const int tid = threadIdx.x;
  double acc = 0.0;
  // partials are loaded eight blocks at a time (clamped, branch-free) and
  // added in block order
  for (int e = tid; e < E; e += 256) {
    double zs = 0.0;
    int64_t c = 0;
    for (int b0 = 0; b0 < nb; b0 += 8) {
      double zv[8];
      int cv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t bb = min(b0 + j, nb - 1);
        zv[j] = pz[bb * E + e];
        cv[j] = pc[bb * E + e];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (b0 + j < nb) {
          zs += zv[j];
          c += cv[j];
        }
    }
    const double zz = zs / (double)T;
    const double yy = (double)c / ((double)T * (double)k);
    counts[e] = (int32_t)c;
    y[e] = (float)yy;
    z[e] = (float)zz;
    acc += yy * zz;
  }
  red[tid] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) {
    double zl = 0.0;
    for (int b0 = 0; b0 < nb; b0 += 8) {
      double lv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) lv[j] = pl[min(b0 + j, nb - 1)];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (b0 + j < nb) zl += lv[j];
    }
    out3[0] = (float)red[0];
    out3[1] = (float)(red[0] * (double)E);
    out3[2] = (float)(zl / (double)T);
  }
}

hipError_t launch_aux_stats(const float* scores, const int32_t* topk, const float* lse, int T,
                            int E, int k, double* pz, int32_t* pc, double* pl, int32_t* counts,
                            float* y, float* z, float* out3, hipStream_t st) {
  const int nb = (T + 255) / 256;
  hipLaunchKernelGGL(aux_partial_kernel, dim3(nb), dim3(256), 0, st, scores, topk, lse, T, E, k,
                     pz, pc, pl);
  hipLaunchKernelGGL(aux_final_kernel, dim3(1), dim3(256), 0, st, pz, pc, pl, nb, T, E, k, counts,
                     y, z, out3);
  return hipGetLastError();
}

// b_e += gamma * sign(1/E - counts_e/(T k)), compared exactly as counts_e*E vs T*k
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts,
                                                          int E, int64_t Tk, float gamma,
                                                          float* __restrict__ bias) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  const int64_t load = (int64_t)counts[e] * E;
  const float step = load < Tk ? 1.0f : (load > Tk ? -1.0f : 0.0f);
  bias[e] = bias[e] + gamma * step;
}

hipError_t launch_bias_update(const int32_t* counts, int E, int64_t Tk, float gamma, float* bias,
                              hipStream_t st) {
  hipLaunchKernelGGL(bias_update_kernel, dim3((E + 255) / 256), dim3(256), 0, st, counts, E, Tk,
                     gamma, bias);
  return hipGetLastError();
}

// -------------------------------------------------------------- permute
// Two launches; the row of every kept assignment is fixed by expert and
// token order, never by thread timing.
// (1) perm_count_kernel, one 1024-thread workgroup: the histogram of the
//     assignments per (block b of bt tokens, expert e) in LDS; per expert,
//     the exclusive prefix of its column over blocks (base[b][e] = tokens
//     before block b routed to e) and its total; totals clipped to the
//     capacity; the exclusive scan of the clipped totals over experts
//     (offsets). base goes to the workspace.
// (2) perm_gather_kernel (below), one wave per token: the rank of each of the
//     token's slots among its expert's assignments is base[b][e] plus the
//     number of earlier tokens of the block routed to e (wave ballots); the
//     slot is kept when the rank is below the capacity, at row
//     offsets[e] + rank; then x[t] is copied to its kept rows.
// bt is the smallest power-of-two multiple of 64 with ceil(T / bt) * E <=
// kPermCells, so the histogram always fits the workgroup's LDS.
constexpr int kPermCells = 32768;   // 128 KiB of int counts

__global__ __launch_bounds__(1024) void perm_count_kernel(const int32_t* __restrict__ topk, int T,
                                                          int E, int k, int bt, int64_t cap,
                                                          int32_t* __restrict__ base,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ n_dropped) {
  __shared__ int h[kPermCells];
  __shared__ int tot[1024];
  __shared__ int sc[1024];
  const int tid = threadIdx.x;
  const int nb = (T + bt - 1) / bt;
  const int cells = nb * E;
  for (int c = tid; c < cells; c += 1024) h[c] = 0;
  __syncthreads();
  for (int t = tid; t < T; t += 1024) {
    const int row = (t / bt) * E;
    for (int j = 0; j < k; ++j) atomicAdd(&h[row + topk[(int64_t)t * k + j]], 1);
  }
  __syncthreads();
  // column prefixes: P threads per expert, each over a chunk of ch blocks
  const int P = 1024 / E;
  const int e = tid / P, part = tid - e * P;
  const int ch = (nb + P - 1) / P;
  const int b0 = part * ch, b1 = min(nb, b0 + ch);
  int s = 0;
  if (e < E)
    for (int b = b0; b < b1; ++b) s += h[b * E + e];
  tot[tid] = s;
  __syncthreads();
  if (e < E) {
    int run = 0;
    for (int q = 0; q < part; ++q) run += tot[e * P + q];
    for (int b = b0; b < b1; ++b) {
      const int v = h[b * E + e];
      h[b * E + e] = run;
      run += v;
    }
    if (part == P - 1) sc[e] = run;   // the expert's total, before the capacity
  }
  __syncthreads();
  int kept = 0;
  if (tid < E) {
    const int n = sc[tid];
    kept = (cap >= 0 && (int64_t)n > cap) ? (int)cap : n;
  }
  __syncthreads();
  sc[tid] = kept;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? sc[tid - o] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  if (tid < E) offsets[tid + 1] = sc[tid];
  if (tid == 0) {
    offsets[0] = 0;
    n_dropped[0] = (int)((int64_t)T * k - sc[E - 1]);
  }
  for (int c = tid; c < cells; c += 1024) base[c] = h[c];
}

int perm_block_tokens(int T, int E) {
  int bt = 64;
  while ((int64_t)((T + bt - 1) / bt) * E > kPermCells) bt *= 2;
  return bt;
}

size_t perm_ws_bytes(int T, int E) {
  const int bt = perm_block_tokens(T, E);
  return (size_t)((T + bt - 1) / bt) * E * 4;
}

// ------------------------------------------------- routed-row streaming
// The permute gather, combine, combine backward and un-permute move rows of
// d elements between token-indexed tensors [T, d] and routed-row tensors
// [T*k, d]. One wave per token (4 tokens per 256-thread workgroup); lane l
// takes 8-element chunks l, l + 64, ... of the row, so each wave instruction
// moves 1 KiB (bf16) of one row. Routed rows go through buffer instructions
// over the whole routed tensor: a dropped slot (row_of = -1) gets an offset
// past the buffer's extent, so its loads return zeros and its stores are
// dropped without touching memory, and every slot's load is issued before
// any of them is used (no branch between a load and the next).
// (check_desc bounds T*k*d*sizeof(T) below 2^31, so byte offsets fit 32 bits.)
template <typename T> struct Rows;
template <> struct Rows<bf16_t> {
  typedef uint4 Packed;
  static __device__ __forceinline__ Packed load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, Packed v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_, v), r, off, 0, 0);
  }
  static __device__ __forceinline__ Packed gload(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  static __device__ __forceinline__ void gstore(bf16_t* p, Packed v) { *reinterpret_cast<uint4*>(p) = v; }
  static __device__ __forceinline__ void unpack(Packed u, float* v) {
    v[0] = bf2f(u.x & 0xffff); v[1] = bf2f(u.x >> 16);
    v[2] = bf2f(u.y & 0xffff); v[3] = bf2f(u.y >> 16);
    v[4] = bf2f(u.z & 0xffff); v[5] = bf2f(u.z >> 16);
    v[6] = bf2f(u.w & 0xffff); v[7] = bf2f(u.w >> 16);
  }
  static __device__ __forceinline__ Packed pack(const float* v) {
    Packed u;
    u.x = pack_bf2(v[0], v[1]); u.y = pack_bf2(v[2], v[3]);
    u.z = pack_bf2(v[4], v[5]); u.w = pack_bf2(v[6], v[7]);
    return u;
  }
};
template <> struct Rows<float> {
  struct Packed { uint4 a, b; };
  static __device__ __forceinline__ Packed load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    Packed p;
    p.a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    p.b = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off == kOOB ? kOOB : off + 16, 0, 0));
    return p;
  }
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, Packed v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_, v.a), r, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_, v.b), r, off == kOOB ? kOOB : off + 16, 0, 0);
  }
  static __device__ __forceinline__ Packed gload(const float* p) {
    Packed v;
    v.a = reinterpret_cast<const uint4*>(p)[0];
    v.b = reinterpret_cast<const uint4*>(p)[1];
    return v;
  }
  static __device__ __forceinline__ void gstore(float* p, Packed v) {
    reinterpret_cast<uint4*>(p)[0] = v.a;
    reinterpret_cast<uint4*>(p)[1] = v.b;
  }
  static __device__ __forceinline__ void unpack(Packed u, float* v) {
    v[0] = __uint_as_float(u.a.x); v[1] = __uint_as_float(u.a.y);
    v[2] = __uint_as_float(u.a.z); v[3] = __uint_as_float(u.a.w);
    v[4] = __uint_as_float(u.b.x); v[5] = __uint_as_float(u.b.y);
    v[6] = __uint_as_float(u.b.z); v[7] = __uint_as_float(u.b.w);
  }
  static __device__ __forceinline__ Packed pack(const float* v) {
    Packed u;
    u.a = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
    u.b = make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7]));
    return u;
  }
};

// byte offset of a token's slot rows (kOOB for a dropped slot or j >= k);
// row_of values are uniform across the wave (scalar loads)
template <typename T, int KM>
__device__ __forceinline__ void slot_rows(const int32_t* __restrict__ row_of, int64_t t, int k,
                                          int64_t d, uint32_t* rb) {
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const int r = j < k ? row_of[t * k + j] : -1;
    rb[j] = r >= 0 ? (uint32_t)((int64_t)r * d * sizeof(T)) : kOOB;
  }
}

// Ranks and rows of token t's slots (see perm_count_kernel), then
// x_perm[row] = x[t] for every kept slot.
template <typename T, int KM>
__global__ __launch_bounds__(256) void perm_gather_kernel(
    const T* __restrict__ x, const int32_t* __restrict__ topk, const int32_t* __restrict__ base,
    const int32_t* __restrict__ offsets, int ntok, int k, int E, int bt, int64_t cap, int64_t d,
    int32_t* __restrict__ row_of, int32_t* __restrict__ token_of, T* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  int ex[KM], cnt[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    ex[j] = j < k ? topk[t * k + j] : -1;
    cnt[j] = 0;
  }
  // earlier tokens of this token's block routed to each of its experts
  const int64_t t0 = (t / bt) * bt;
  for (int64_t s0 = t0; s0 < t; s0 += 64) {
    const int64_t tt = s0 + lane;
    const bool valid = tt < t;
    int me[KM];
#pragma unroll
    for (int jj = 0; jj < KM; ++jj) me[jj] = (valid && jj < k) ? topk[tt * k + jj] : -2;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      bool m = false;
#pragma unroll
      for (int jj = 0; jj < KM; ++jj) m = m || me[jj] == ex[j];
      cnt[j] += __popcll(__ballot(m && j < k));
    }
  }
  uint32_t rb[KM];
  int myrow = -1;
  const int32_t* brow = base + (t / bt) * E;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    int row = -1;
    if (j < k) {
      const int64_t rank = (int64_t)brow[ex[j]] + cnt[j];
      if (cap < 0 || rank < cap) row = offsets[ex[j]] + (int)rank;
    }
    rb[j] = row >= 0 ? (uint32_t)((int64_t)row * d * sizeof(T)) : kOOB;
    if (lane == j) myrow = row;
  }
  if (lane < k) {
    row_of[t * k + lane] = myrow;
    if (myrow >= 0) token_of[myrow] = (int32_t)t;
  }
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(x_perm, (int64_t)ntok * k * d * sizeof(T));
  const T* xr = x + t * d;
  for (int64_t c = lane; c < d / 8; c += 64) {
    const typename Rows<T>::Packed v = Rows<T>::gload(xr + c * 8);
    const uint32_t co = (uint32_t)(c * 8 * sizeof(T));
#pragma unroll
    for (int j = 0; j < KM; ++j) Rows<T>::store(rp, rb[j] == kOOB ? kOOB : rb[j] + co, v);
  }
}

hipError_t launch_permute(const void* x, bool bf16, const int32_t* topk, int T, int E, int k,
                          int64_t d, int64_t cap, int32_t* base, int32_t* offsets,
                          int32_t* row_of, int32_t* token_of, int32_t* n_dropped, void* x_perm,
                          hipStream_t st) {
  const int bt = perm_block_tokens(T, E);
  hipLaunchKernelGGL(perm_count_kernel, dim3(1), dim3(1024), 0, st, topk, T, E, k, bt, cap, base,
                     offsets, n_dropped);
  const dim3 grid((T + 3) / 4), block(256);
#define MOE_GATHER(TY, KM)                                                                     \
  hipLaunchKernelGGL((perm_gather_kernel<TY, KM>), grid, block, 0, st, (const TY*)x, topk, base, \
                     offsets, T, k, E, bt, cap, d, row_of, token_of, (TY*)x_perm)
  if (bf16) {
    if (k <= 2) MOE_GATHER(bf16_t, 2);
    else if (k <= 8) MOE_GATHER(bf16_t, 8);
    else MOE_GATHER(bf16_t, 16);
  } else {
    if (k <= 2) MOE_GATHER(float, 2);
    else if (k <= 8) MOE_GATHER(float, 8);
    else MOE_GATHER(float, 16);
  }
#undef MOE_GATHER
  return hipGetLastError();
}

// -------------------------------------------------------------- combine
// y[t] = out_shared[t] + sum_j gate[t,j] * out[row_of[t,j]] (slot order,
// float32, one rounding); a dropped slot adds nothing.
template <typename T, int KM>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ out,
                                                      const T* __restrict__ out_shared,
                                                      const float* __restrict__ gate,
                                                      const int32_t* __restrict__ row_of, int ntok,
                                                      int k, int64_t d, T* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(out, (int64_t)ntok * k * d * sizeof(T));
  uint32_t rb[KM];
  float g[KM];
  slot_rows<T, KM>(row_of, t, k, d, rb);
#pragma unroll
  for (int j = 0; j < KM; ++j) g[j] = j < k ? gate[t * k + j] : 0.f;
  for (int64_t c = lane; c < d / 8; c += 64) {
    const uint32_t co = (uint32_t)(c * 8 * sizeof(T));
    typename Rows<T>::Packed pv[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) pv[j] = Rows<T>::load(ro, rb[j] == kOOB ? kOOB : rb[j] + co);
    float acc[8], v[8];
    if (out_shared) {
      Rows<T>::unpack(Rows<T>::gload(out_shared + t * d + c * 8), acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      Rows<T>::unpack(pv[j], v);
      const bool kept = rb[j] != kOOB;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = kept ? fmaf(g[j], v[i], acc[i]) : acc[i];
    }
    Rows<T>::gstore(y + t * d + c * 8, Rows<T>::pack(acc));
  }
}

// dgate[t,j] = <dy[t], out[row]>, dout[row] = gate * dy[t]. Each lane keeps
// one partial per slot (chunks in ascending order, an fma chain inside a
// chunk); the wave's partials are then summed by a fixed butterfly.
template <typename T, int KM>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T* __restrict__ dy,
                                                          const T* __restrict__ out,
                                                          const float* __restrict__ gate,
                                                          const int32_t* __restrict__ row_of,
                                                          int ntok, int k, int64_t d,
                                                          float* __restrict__ dgate,
                                                          T* __restrict__ dout) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const int64_t bytes = (int64_t)ntok * k * d * sizeof(T);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(out, bytes);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(dout, bytes);
  uint32_t rb[KM];
  float g[KM], part[KM];
  slot_rows<T, KM>(row_of, t, k, d, rb);
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    g[j] = j < k ? gate[t * k + j] : 0.f;
    part[j] = 0.f;
  }
  for (int64_t c = lane; c < d / 8; c += 64) {
    const uint32_t co = (uint32_t)(c * 8 * sizeof(T));
    typename Rows<T>::Packed pv[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) pv[j] = Rows<T>::load(ro, rb[j] == kOOB ? kOOB : rb[j] + co);
    float vy[8], vo[8], w[8];
    Rows<T>::unpack(Rows<T>::gload(dy + t * d + c * 8), vy);
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      Rows<T>::unpack(pv[j], vo);
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p = fmaf(vy[i], vo[i], p);
        w[i] = g[j] * vy[i];
      }
      part[j] += p;
      Rows<T>::store(rd, rb[j] == kOOB ? kOOB : rb[j] + co, Rows<T>::pack(w));
    }
  }
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < k) {   // k is uniform: every lane of the wave takes the same branch
      const float sj = wave_sum(part[j]);
      if (lane == 0) dgate[t * k + j] = rb[j] == kOOB ? 0.f : sj;
    }
  }
}

// dx[t] = dx_shared[t] + sum_j dx_perm[row_of[t,j]] + dx_router[t]; one rounding.
template <typename T, int KM>
__global__ __launch_bounds__(256) void unpermute_kernel(const T* __restrict__ dx_perm,
                                                        const int32_t* __restrict__ row_of,
                                                        const T* __restrict__ dx_shared,
                                                        const float* __restrict__ dx_router,
                                                        int ntok, int k, int64_t d,
                                                        T* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(dx_perm, (int64_t)ntok * k * d * sizeof(T));
  uint32_t rb[KM];
  slot_rows<T, KM>(row_of, t, k, d, rb);
  for (int64_t c = lane; c < d / 8; c += 64) {
    const uint32_t co = (uint32_t)(c * 8 * sizeof(T));
    typename Rows<T>::Packed pv[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) pv[j] = Rows<T>::load(rp, rb[j] == kOOB ? kOOB : rb[j] + co);
    float acc[8], v[8];
    if (dx_shared) {
      Rows<T>::unpack(Rows<T>::gload(dx_shared + t * d + c * 8), acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      Rows<T>::unpack(pv[j], v);
      const bool kept = rb[j] != kOOB;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = kept ? acc[i] + v[i] : acc[i];
    }
    if (dx_router) {
      Vec8<float>::load(dx_router + t * d + c * 8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    Rows<T>::gstore(dx + t * d + c * 8, Rows<T>::pack(acc));
  }
}

// the smallest slot count instantiated that holds k (k <= 16)
#define MOE_BY_K(MAC, TY)            \
  do {                               \
    if (k <= 1) MAC(TY, 1);          \
    else if (k <= 2) MAC(TY, 2);     \
    else if (k <= 4) MAC(TY, 4);     \
    else if (k <= 8) MAC(TY, 8);     \
    else MAC(TY, 16);                \
  } while (0)

hipError_t launch_combine(const void* out, const void* out_shared, bool bf16, const float* gate,
                          const int32_t* row_of, int T, int k, int64_t d, void* y, hipStream_t st) {
  const dim3 grid((T + 3) / 4), block(256);
#define MOE_COMB(TY, KM)                                                                        \
  hipLaunchKernelGGL((combine_kernel<TY, KM>), grid, block, 0, st, (const TY*)out,             \
                     (const TY*)out_shared, gate, row_of, T, k, d, (TY*)y)
  if (bf16) MOE_BY_K(MOE_COMB, bf16_t);
  else MOE_BY_K(MOE_COMB, float);
#undef MOE_COMB
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const void* dy, const void* out, bool bf16, const float* gate,
                              const int32_t* row_of, int T, int k, int64_t d, float* dgate,
                              void* dout, hipStream_t st) {
  const dim3 grid((T + 3) / 4), block(256);
#define MOE_CBWD(TY, KM)                                                                        \
  hipLaunchKernelGGL((combine_bwd_kernel<TY, KM>), grid, block, 0, st, (const TY*)dy,          \
                     (const TY*)out, gate, row_of, T, k, d, dgate, (TY*)dout)
  if (bf16) MOE_BY_K(MOE_CBWD, bf16_t);
  else MOE_BY_K(MOE_CBWD, float);
#undef MOE_CBWD
  return hipGetLastError();
}

hipError_t launch_unpermute(const void* dx_perm, const int32_t* row_of, const void* dx_shared,
                            const float* dx_router, bool bf16, int T, int k, int64_t d, void* dx,
                            hipStream_t st) {
  const dim3 grid((T + 3) / 4), block(256);
#define MOE_UNP(TY, KM)                                                                         \
  hipLaunchKernelGGL((unpermute_kernel<TY, KM>), grid, block, 0, st, (const TY*)dx_perm,       \
                     row_of, (const TY*)dx_shared, dx_router, T, k, d, (TY*)dx)
  if (bf16) MOE_BY_K(MOE_UNP, bf16_t);
  else MOE_BY_K(MOE_UNP, float);
#undef MOE_UNP
  return hipGetLastError();
}
#undef MOE_BY_K

// ------------------------------------------------------- router backward
// One wave per token: dlogits[t, :] from the renormalised-gate gradient and
// the optional aux term (y held fixed).
template <int EPL>
__global__ __launch_bounds__(256) void router_dlogits_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ topk,
    const float* __restrict__ gate, const float* __restrict__ dgate, const float* __restrict__ y,
    float aux_coef, const float* __restrict__ lse, float z_coef, float inv_tau, int T, int E,
    int k, int score, float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float inner = 0.f, ssum = 0.f;
  for (int j = 0; j < k; ++j) {
    inner = fmaf(gate[t * k + j], dgate[t * k + j], inner);
    ssum += scores[t * E + topk[t * k + j]];
  }
  float s[EPL], out[EPL];
  float ys = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    s[i] = e < E ? scores[t * E + e] : 0.f;
    out[i] = 0.f;
    if (aux_coef != 0.f && e < E) ys = fmaf(y[e], s[i], ys);
  }
  if (aux_coef != 0.f && score == 0) ys = wave_sum(ys);
  for (int j = 0; j < k; ++j) {
    const int e = topk[t * k + j];
    const float g = gate[t * k + j], dg = dgate[t * k + j];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (lane + 64 * i != e) continue;
      if (score == 0) out[i] = g * (dg - inner);
      else out[i] = s[i] * (1.f - s[i]) * (dg - inner) / ssum;
    }
  }
  const float c = aux_coef * (float)E / (float)T;
  // z-loss term; only softmax scoring takes it, where the scores are softmax(logits)
  const float zc = z_coef != 0.f ? z_coef * 2.0f / (float)T * lse[t] : 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e >= E) continue;
    if (aux_coef != 0.f) {
      if (score == 0) out[i] += c * s[i] * (y[e] - ys);
      else out[i] += c * y[e] * s[i] * (1.f - s[i]);
    }
    if (z_coef != 0.f) out[i] += zc * s[i];
    dl[t * E + e] = out[i] * inv_tau;
  }
}

hipError_t launch_router_dlogits(const float* scores, const int32_t* topk, const float* gate,
                                 const float* dgate, const float* y, float aux_coef,
                                 const float* lse, float z_coef, float inv_tau, int T, int E, int k,
                                 int score, float* dl, hipStream_t st) {
  dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(router_dlogits_kernel<1>, grid, block, 0, st, scores, topk, gate, dgate, y, aux_coef, lse, z_coef, inv_tau, T, E, k, score, dl);
  else if (E <= 128)
    hipLaunchKernelGGL(router_dlogits_kernel<2>, grid, block, 0, st, scores, topk, gate, dgate, y, aux_coef, lse, z_coef, inv_tau, T, E, k, score, dl);
  else if (E <= 256)
    hipLaunchKernelGGL(router_dlogits_kernel<4>, grid, block, 0, st, scores, topk, gate, dgate, y, aux_coef, lse, z_coef, inv_tau, T, E, k, score, dl);
  else
    hipLaunchKernelGGL(router_dlogits_kernel<16>, grid, block, 0, st, scores, topk, gate, dgate, y, aux_coef, lse, z_coef, inv_tau, T, E, k, score, dl);
  return hipGetLastError();
}

// dx_router[t] = sum_j dl[t, e_j] W_r[e_j] when dl is zero off the chosen
// experts (no aux term): a k-row gather of W_r per token.
__global__ __launch_bounds__(256) void router_dx_sparse_kernel(const float* __restrict__ dl,
                                                               const int32_t* __restrict__ topk,
                                                               const float* __restrict__ w_r,
                                                               int E, int k, int64_t d,
                                                               float* __restrict__ dx) {
  const int64_t t = blockIdx.x;
  int es[16];
  float c[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    es[j] = j < k ? topk[t * k + j] : -1;
    c[j] = j < k ? dl[t * E + es[j]] : 0.f;
  }
  for (int64_t col = threadIdx.x * 8; col < d; col += 256 * 8) {
    float acc[8], v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (es[j] < 0) continue;
      Vec8<float>::load(w_r + (int64_t)es[j] * d + col, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(c[j], v[i], acc[i]);
    }
    Vec8<float>::store(dx + t * d + col, acc);
  }
}

hipError_t launch_router_dx_sparse(const float* dl, const int32_t* topk, const float* w_r, int T,
                                   int E, int k, int64_t d, float* dx, hipStream_t st) {
  hipLaunchKernelGGL(router_dx_sparse_kernel, dim3(T), dim3(256), 0, st, dl, topk, w_r, E, k, d, dx);
  return hipGetLastError();
}

// zero n 16-byte words (a kernel, so the call stays graph-capturable)
__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  int64_t nb = (n + 255) / 256;
  if (nb > 65536) nb = 65536;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)nb), dim3(256), 0, st, (uint4*)p, n);
  return hipGetLastError();
}

// out[i] = sum_s part[s][i], s ascending
// dW_r = dl^T x for few experts (E <= 8): a streaming reduction over tokens,
// x read once. Block (bx, chunk) is one wave over 512 columns (8 per lane,
// one 16-byte load per token); it sums, over the chunk's kRdwTok tokens in
// ascending order, dl[t][e] * x[t][c .. c+7], with the rows of 8 tokens
// loaded ahead of their FMAs. The partial [chunk][E][d] is folded by
// splitk_reduce_kernel in chunk order, so the result is deterministic.
constexpr int kRdwTok = 64;
constexpr int kRdwEMax = 8;
constexpr int kRdwAhead = 8;

template <typename TX>
__global__ __launch_bounds__(64) void router_dw_small_kernel(const float* __restrict__ dl,
                                                             const TX* __restrict__ x, int T,
                                                             int E, int64_t d,
                                                             float* __restrict__ part) {
  __shared__ float sdl[kRdwTok * kRdwEMax];
  const int chunk = blockIdx.y, lane = threadIdx.x;
  const int t0 = chunk * kRdwTok;
  const int nt = T - t0 < kRdwTok ? T - t0 : kRdwTok;
  // weights of the chunk's tokens, zero past its end and for e >= E, so the
  // loop below has no branches (the loads stay in flight together)
  for (int i = lane; i < kRdwTok * kRdwEMax; i += 64) {
    const int tt = i / kRdwEMax, e = i - tt * kRdwEMax;
    sdl[i] = (tt < nt && e < E) ? dl[(int64_t)(t0 + tt) * E + e] : 0.f;
  }
  __syncthreads();
  const int64_t c = ((int64_t)blockIdx.x * 64 + lane) * 8;
  if (c >= d) return;
  float acc[kRdwEMax][8];
#pragma unroll
  for (int e = 0; e < kRdwEMax; ++e)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[e][j] = 0.f;
  const TX* xr = x + (int64_t)t0 * d + c;
  for (int tb = 0; tb < nt; tb += kRdwAhead) {
    float xv[kRdwAhead][8];
#pragma unroll
    for (int u = 0; u < kRdwAhead; ++u) {
      const int tt = tb + u < nt ? tb + u : nt - 1;   // in range; its weight is 0 past nt
      Vec8<TX>::load(xr + (int64_t)tt * d, xv[u]);
    }
#pragma unroll
    for (int u = 0; u < kRdwAhead; ++u)
#pragma unroll
      for (int e = 0; e < kRdwEMax; ++e) {
        const float w = sdl[(tb + u) * kRdwEMax + e];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[e][j] = fmaf(w, xv[u][j], acc[e][j]);
      }
  }
  for (int e = 0; e < E; ++e) Vec8<float>::store(part + ((int64_t)chunk * E + e) * d + c, acc[e]);
}

hipError_t launch_router_dw_small(const float* dl, const void* x, bool x_bf16, int T, int E,
                                  int64_t d, float* part, hipStream_t st) {
  if (E > kRdwEMax || T <= 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((d + 511) / 512), (unsigned)((T + kRdwTok - 1) / kRdwTok));
  if (x_bf16)
    hipLaunchKernelGGL(router_dw_small_kernel<bf16_t>, grid, dim3(64), 0, st, dl,
                       (const bf16_t*)x, T, E, d, part);
  else
    hipLaunchKernelGGL(router_dw_small_kernel<float>, grid, dim3(64), 0, st, dl,
                       (const float*)x, T, E, d, part);
  return hipGetLastError();
}

int router_dw_small_chunks(int T) { return (T + kRdwTok - 1) / kRdwTok; }

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int S, int64_t n,
                                                            float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  // partials summed in index order; loads issued eight at a time
  float acc = 0.f;
  int s = 0;
  for (; s + 8 <= S; s += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(s + u) * n + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; s < S; ++s) acc += part[(int64_t)s * n + i];
  out[i] = acc;
}

hipError_t launch_splitk_reduce(const float* part, int S, int64_t n, float* out, hipStream_t st) {
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     part, S, n, out);
  return hipGetLastError();
}

// ------------------------------------------- router products on bf16 matrix cores
// A float32 value v splits exactly into three bf16 terms, v = hi + mid + lo:
// hi = bf16(v) leaves a remainder of at most 16 significant bits (exact in
// float32), mid = bf16 of that remainder leaves at most 8, which lo then holds
// exactly (round to nearest even at every step; values near the bottom of the
// float32 range, where lo would be subnormal, are the exception and do not
// arise for router weights or logit gradients). With x in bf16, every product
// x * hi, x * mid, x * lo is exact in float32, so a bf16 MFMA GEMM over the
// three terms, accumulated in float32, is a float32 product of x and the
// float32 operand. Block j (0 <= j < nb) of element (r, c) is
// dst[r * ldd + j * sst + c] and holds term (code >> 2j) & 3 (0 hi, 1 mid,
// 2 lo): code 0x24 writes hi, mid, lo to blocks 0, 1, 2.
__global__ __launch_bounds__(256) void split_bf16x3_kernel(const float* __restrict__ src, int64_t rows,
                                                           int64_t cols, bf16_t* __restrict__ dst,
                                                           int64_t ldd, int64_t sst, int nb, int code) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 4-column group
  const int64_t cq = cols >> 2;
  if (q >= rows * cq) return;
  const int64_t r = q / cq, c = (q - r * cq) << 2;
  const float4 v = *reinterpret_cast<const float4*>(src + r * cols + c);
  const float in[4] = {v.x, v.y, v.z, v.w};
  uint32_t t[3][4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t h = f2bf(in[e]);
    const float r1 = in[e] - bf2f(h);
    const uint32_t m = f2bf(r1);
    const float r2 = r1 - bf2f(m);
    t[0][e] = h;
    t[1][e] = m;
    t[2][e] = f2bf(r2);
  }
  uint2 w[3];
#pragma unroll
  for (int sp = 0; sp < 3; ++sp) {
    w[sp].x = t[sp][0] | (t[sp][1] << 16);
    w[sp].y = t[sp][2] | (t[sp][3] << 16);
  }
  for (int j = 0; j < nb; ++j) {
    const int sp = (code >> (2 * j)) & 3;
    *reinterpret_cast<uint2*>(dst + r * ldd + j * sst + c) = sp == 0 ? w[0] : (sp == 1 ? w[1] : w[2]);
  }
}

hipError_t launch_split_bf16x3(const float* src, int64_t rows, int64_t cols, bf16_t* dst, int64_t ldd,
                               int64_t sst, hipStream_t st, int nb, int code) {
  const int64_t n = rows * (cols >> 2);
  if (n == 0) return hipSuccess;
  if (nb < 1 || nb > 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(split_bf16x3_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src,
                     rows, cols, dst, ldd, sst, nb, code);
  return hipGetLastError();
}

// out[r * cols + c] = bias[c] (if any) + sum over partitions g = 0..S-1 of
// ((lo + mid) + hi), the three split products of partition g at
// part[g * gst + s * sst + r * ld + c] (s = 0 hi, 1 mid, 2 lo); a fixed order.
__global__ __launch_bounds__(256) void fold_bf16x3_kernel(const float* __restrict__ part, int S,
                                                          int64_t gst, int64_t sst, int64_t ld,
                                                          int64_t rows, int64_t cols,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t cq = cols >> 2;
  if (q >= rows * cq) return;
  const int64_t r = q / cq, c = (q - r * cq) << 2;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int g = 0; g < S; ++g) {
    const float* b = part + g * gst + r * ld + c;
    const float4 h = *reinterpret_cast<const float4*>(b);
    const float4 m = *reinterpret_cast<const float4*>(b + sst);
    const float4 l = *reinterpret_cast<const float4*>(b + 2 * sst);
    acc.x += (l.x + m.x) + h.x;
    acc.y += (l.y + m.y) + h.y;
    acc.z += (l.z + m.z) + h.z;
    acc.w += (l.w + m.w) + h.w;
  }
  if (bias) {
    acc.x += bias[c]; acc.y += bias[c + 1]; acc.z += bias[c + 2]; acc.w += bias[c + 3];
  }
  *reinterpret_cast<float4*>(out + r * cols + c) = acc;
}

hipError_t launch_fold_bf16x3(const float* part, int S, int64_t gst, int64_t sst, int64_t ld,
                              int64_t rows, int64_t cols, const float* bias, float* out,
                              hipStream_t st) {
  const int64_t n = rows * (cols >> 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fold_bf16x3_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, S,
                     gst, sst, ld, rows, cols, bias, out);
  return hipGetLastError();
}

}  // namespace moe
