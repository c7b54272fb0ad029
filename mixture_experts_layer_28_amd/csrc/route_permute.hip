// Router top-k, load-balance statistics, permute (local dispatch), combine,
// and their backward companions. All HBM-bound or latency-bound; each is a
// plain streaming kernel with 16-byte accesses and fixed reduction orders.
#include "gemm_tile.h"

namespace moe {

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
// 64-token blocks. (1) per-block histogram; (2) per expert, exclusive scan
// over blocks (in place) and capacity-clipped exclusive scan over experts;
// (3) per block, rank of each assignment among earlier tokens of the block
// routed to the same expert (wave ballot), giving its row.
__global__ __launch_bounds__(64) void perm_hist_kernel(const int32_t* __restrict__ topk, int T,
                                                       int E, int k, int32_t* __restrict__ hist) {
  __shared__ int h[1024];
  const int b = blockIdx.x, lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) h[e] = 0;
  __syncthreads();
  const int t = b * 64 + lane;
  if (t < T)
    for (int j = 0; j < k; ++j) atomicAdd(&h[topk[(int64_t)t * k + j]], 1);
  __syncthreads();
  for (int e = lane; e < E; e += 64) hist[(int64_t)b * E + e] = h[e];
}

__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t* __restrict__ hist, int nb, int T,
                                                         int E, int k, int64_t cap,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ n_dropped) {
  __shared__ int sc[1024];
  const int tid = threadIdx.x;
  int kept = 0;
  if (tid < E) {
    // 16 block counts are loaded before any is replaced (clamped, so the
    // loads need no branch), then the running sum is written back.
    int run = 0;
    for (int b0 = 0; b0 < nb; b0 += 16) {
      int v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int bb = min(b0 + j, nb - 1);
        const int h = hist[(int64_t)bb * E + tid];
        v[j] = b0 + j < nb ? h : 0;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (b0 + j < nb) hist[(int64_t)(b0 + j) * E + tid] = run;
        run += v[j];
      }
    }
    kept = (cap >= 0 && (int64_t)run > cap) ? (int)cap : run;
  }
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
    n_dropped[0] = T * k - sc[E - 1];
  }
}

__global__ __launch_bounds__(64) void perm_rank_kernel(const int32_t* __restrict__ topk, int T,
                                                       int E, int k, int64_t cap,
                                                       const int32_t* __restrict__ base,
                                                       const int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ row_of,
                                                       int32_t* __restrict__ token_of) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int t = b * 64 + lane;
  int mine[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) mine[j] = (t < T && j < k) ? topk[(int64_t)t * k + j] : -1;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int e = 0; e < E; ++e) {
    int slot = -1;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (mine[j] == e) slot = j;
    const uint64_t m = __ballot(slot >= 0);
    if (m == 0) continue;
    if (slot >= 0) {
      const int64_t rank = (int64_t)base[(int64_t)b * E + e] + __popcll(m & lt);
      if (cap < 0 || rank < cap) {
        const int row = offsets[e] + (int)rank;
        row_of[(int64_t)t * k + slot] = row;
        token_of[row] = t;
      } else {
        row_of[(int64_t)t * k + slot] = -1;
      }
    }
  }
}

// One block per token: read x[t] once, write it to each kept row.
template <typename T>
__global__ __launch_bounds__(256) void perm_gather_kernel(const T* __restrict__ x,
                                                          const int32_t* __restrict__ row_of,
                                                          int k, int64_t d,
                                                          T* __restrict__ x_perm) {
  const int64_t t = blockIdx.x;
  int rows[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) rows[j] = j < k ? row_of[t * k + j] : -1;
  constexpr int EL = 16 / sizeof(T);
  const int64_t nch = d / EL;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * d);
  for (int64_t c = threadIdx.x; c < nch; c += 256) {
    const uint4 v = src[c];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (rows[j] >= 0) reinterpret_cast<uint4*>(x_perm + (int64_t)rows[j] * d)[c] = v;
  }
}

hipError_t launch_permute(const void* x, bool bf16, const int32_t* topk, int T, int E, int k,
                          int64_t d, int64_t cap, int32_t* hist, int32_t* offsets,
                          int32_t* row_of, int32_t* token_of, int32_t* n_dropped, void* x_perm,
                          hipStream_t st) {
  const int nb = (T + 63) / 64;
  hipLaunchKernelGGL(perm_hist_kernel, dim3(nb), dim3(64), 0, st, topk, T, E, k, hist);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, st, hist, nb, T, E, k, cap, offsets, n_dropped);
  hipLaunchKernelGGL(perm_rank_kernel, dim3(nb), dim3(64), 0, st, topk, T, E, k, cap, hist, offsets, row_of, token_of);
  if (bf16)
    hipLaunchKernelGGL(perm_gather_kernel<bf16_t>, dim3(T), dim3(256), 0, st,
                       (const bf16_t*)x, row_of, k, d, (bf16_t*)x_perm);
  else
    hipLaunchKernelGGL(perm_gather_kernel<float>, dim3(T), dim3(256), 0, st,
                       (const float*)x, row_of, k, d, (float*)x_perm);
  return hipGetLastError();
}

// -------------------------------------------------------------- combine
// y[t] = out_shared[t] + sum_j gate[t,j] * out[row_of[t,j]] (slot order).
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ out,
                                                      const T* __restrict__ out_shared,
                                                      const float* __restrict__ gate,
                                                      const int32_t* __restrict__ row_of, int k,
                                                      int64_t d, T* __restrict__ y) {
  const int64_t t = blockIdx.x;
  int rows[16];
  float g[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    rows[j] = j < k ? row_of[t * k + j] : -1;
    g[j] = j < k ? gate[t * k + j] : 0.f;
  }
  for (int64_t c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float acc[8], v[8];
    if (out_shared) {
      Vec8<T>::load(out_shared + t * d + c, acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (rows[j] < 0) continue;
      Vec8<T>::load(out + (int64_t)rows[j] * d + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(g[j], v[i], acc[i]);
    }
    Vec8<T>::store(y + t * d + c, acc);
  }
}

// dgate[t,j] = <dy[t], out[row]>, dout[row] = gate * dy[t]; one block per token.
template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T* __restrict__ dy,
                                                          const T* __restrict__ out,
                                                          const float* __restrict__ gate,
                                                          const int32_t* __restrict__ row_of,
                                                          int k, int64_t d,
                                                          float* __restrict__ dgate,
                                                          T* __restrict__ dout) {
  __shared__ float red[4][16];
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int rows[16];
  float g[16], part[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    rows[j] = j < k ? row_of[t * k + j] : -1;
    g[j] = j < k ? gate[t * k + j] : 0.f;
    part[j] = 0.f;
  }
  for (int64_t c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float vy[8], vo[8], w[8];
    Vec8<T>::load(dy + t * d + c, vy);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (rows[j] < 0) continue;
      Vec8<T>::load(out + (int64_t)rows[j] * d + c, vo);
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p = fmaf(vy[i], vo[i], p);
        w[i] = g[j] * vy[i];
      }
      part[j] += p;
      Vec8<T>::store(dout + (int64_t)rows[j] * d + c, w);
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j >= k) break;
    const float s = wave_sum(part[j]);
    if (lane == 0) red[wave][j] = s;
  }
  __syncthreads();
  if (threadIdx.x < k) {
    const int j = threadIdx.x;
    dgate[t * k + j] = rows[j] < 0 ? 0.f : ((red[0][j] + red[1][j]) + (red[2][j] + red[3][j]));
  }
}

// dx[t] = dx_shared[t] + sum_j dx_perm[row_of[t,j]] + dx_router[t]; one rounding.
template <typename T>
__global__ __launch_bounds__(256) void unpermute_kernel(const T* __restrict__ dx_perm,
                                                        const int32_t* __restrict__ row_of,
                                                        const T* __restrict__ dx_shared,
                                                        const float* __restrict__ dx_router,
                                                        int k, int64_t d, T* __restrict__ dx) {
  const int64_t t = blockIdx.x;
  int rows[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) rows[j] = j < k ? row_of[t * k + j] : -1;
  for (int64_t c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float acc[8], v[8];
    if (dx_shared) {
      Vec8<T>::load(dx_shared + t * d + c, acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (rows[j] < 0) continue;
      Vec8<T>::load(dx_perm + (int64_t)rows[j] * d + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if (dx_router) {
      Vec8<float>::load(dx_router + t * d + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    Vec8<T>::store(dx + t * d + c, acc);
  }
}

hipError_t launch_combine(const void* out, const void* out_shared, bool bf16, const float* gate,
                          const int32_t* row_of, int T, int k, int64_t d, void* y, hipStream_t st) {
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(T), dim3(256), 0, st, (const bf16_t*)out,
                       (const bf16_t*)out_shared, gate, row_of, k, d, (bf16_t*)y);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(T), dim3(256), 0, st, (const float*)out,
                       (const float*)out_shared, gate, row_of, k, d, (float*)y);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const void* dy, const void* out, bool bf16, const float* gate,
                              const int32_t* row_of, int T, int k, int64_t d, float* dgate,
                              void* dout, hipStream_t st) {
  if (bf16)
    hipLaunchKernelGGL(combine_bwd_kernel<bf16_t>, dim3(T), dim3(256), 0, st, (const bf16_t*)dy,
                       (const bf16_t*)out, gate, row_of, k, d, dgate, (bf16_t*)dout);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<float>, dim3(T), dim3(256), 0, st, (const float*)dy,
                       (const float*)out, gate, row_of, k, d, dgate, (float*)dout);
  return hipGetLastError();
}

hipError_t launch_unpermute(const void* dx_perm, const int32_t* row_of, const void* dx_shared,
                            const float* dx_router, bool bf16, int T, int k, int64_t d, void* dx,
                            hipStream_t st) {
  if (bf16)
    hipLaunchKernelGGL(unpermute_kernel<bf16_t>, dim3(T), dim3(256), 0, st,
                       (const bf16_t*)dx_perm, row_of, (const bf16_t*)dx_shared, dx_router, k, d,
                       (bf16_t*)dx);
  else
    hipLaunchKernelGGL(unpermute_kernel<float>, dim3(T), dim3(256), 0, st, (const float*)dx_perm,
                       row_of, (const float*)dx_shared, dx_router, k, d, (float*)dx);
  return hipGetLastError();
}

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

}  // namespace moe
