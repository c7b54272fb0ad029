// C ABI of libmoe (declared in include/moe.h): argument validation before any
// HIP call, workspace layout, and the ordered kernel launches of each call.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "common.h"

#include <algorithm>

namespace moe {
hipError_t gemm_bf16(const GemmArgs& p, bool akm, bool bkm, int epi, int rag, hipStream_t s);
hipError_t launch_quant_fp8_blocks(const void* src, int64_t rows, int64_t K, int64_t ld_src,
                                   const int32_t* valid_rows, void* codes, int64_t ld_q,
                                   uint8_t* scales, hipStream_t st, int fmt = 0);
hipError_t launch_quant_fp8_squares(const void* src, int64_t G, int64_t R, int64_t C, void* codes,
                                    uint8_t* scales, void* codes_t, uint8_t* scales_t, hipStream_t st);
hipError_t launch_quant_fp8_tblocks(const void* src, int64_t R, int64_t C, const int32_t* off, int G,
                                    int32_t* tab, void* codes_t, uint8_t* scales, hipStream_t st,
                                    int fmt = 0, void* rcodes = nullptr, uint8_t* rscales = nullptr);
hipError_t launch_set_bounds(int32_t* bounds, int32_t lo, int32_t hi, hipStream_t st);
hipError_t gemm_f32(const GemmArgs& p, bool akm, bool bkm, int epi, int rag, hipStream_t s);
hipError_t gemm_fp8(const GemmArgs& p, int epi, int rag, hipStream_t s, int a_fmt = 0);
hipError_t launch_quant_fp8_t(const void*, int64_t, int64_t, int64_t, void*, int32_t*, hipStream_t);
hipError_t launch_quant_fp8_both(const void*, int64_t, int64_t, int64_t, void*, int32_t*, void*,
                                 int32_t*, void*, hipStream_t);
size_t quant_fp8_both_ws(int64_t, int64_t, int64_t);
hipError_t launch_quant_fp8(const void*, int64_t, int64_t, int64_t, const int32_t*, void*, int64_t,
                            int32_t*, hipStream_t, int fmt = 0);
hipError_t gemm_router_logits(const GemmArgs& p, bool x_bf16, hipStream_t s);
hipError_t gemm_router_dw(const GemmArgs& p, bool x_bf16, hipStream_t s);
hipError_t gemm_router_dx(const GemmArgs& p, hipStream_t s);
hipError_t launch_router_topk(const float*, int, int, int, int, const float*, int32_t*, float*,
                              float*, float*, const float*, float, hipStream_t);
hipError_t launch_aux_stats(const float*, const int32_t*, const float*, int, int, int, double*,
                            int32_t*, double*, int32_t*, float*, float*, float*, hipStream_t);
hipError_t launch_bias_update(const int32_t*, int, int64_t, float, float*, hipStream_t);
hipError_t launch_permute(const void*, bool, const int32_t*, int, int, int, int64_t, int64_t,
                          int32_t*, int32_t*, int32_t*, int32_t*, int32_t*, void*, hipStream_t);
hipError_t launch_combine(const void*, const void*, bool, const float*, const int32_t*, int, int,
                          int64_t, void*, hipStream_t);
hipError_t launch_combine_bwd(const void*, const void*, bool, const float*, const int32_t*, int,
                              int, int64_t, float*, void*, hipStream_t);
hipError_t launch_unpermute(const void*, const int32_t*, const void*, const float*, bool, int, int,
                            int64_t, void*, hipStream_t);
hipError_t launch_router_dlogits(const float*, const int32_t*, const float*, const float*,
                                 const float*, float, const float*, float, float, int, int, int,
                                 int, float*, hipStream_t);
hipError_t launch_router_dx_sparse(const float*, const int32_t*, const float*, int, int, int,
                                   int64_t, float*, hipStream_t);
hipError_t launch_splitk_reduce(const float*, int, int64_t, float*, hipStream_t);
hipError_t launch_split_bf16x3(const float*, int64_t, int64_t, bf16_t*, int64_t, int64_t, hipStream_t,
                               int nb = 3, int code = 0x24);
hipError_t launch_fold_bf16x3(const float*, int, int64_t, int64_t, int64_t, int64_t, int64_t,
                              const float*, float*, hipStream_t);
hipError_t gemm_bf16(const GemmArgs& p, bool akm, bool bkm, int epi, int rag, hipStream_t s);
hipError_t launch_router_dw_small(const float*, const void*, bool, int, int, int64_t, float*,
                                  hipStream_t);
int router_dw_small_chunks(int T);
size_t perm_ws_bytes(int T, int E);
hipError_t launch_fill_zero(void*, size_t, hipStream_t);
hipError_t launch_router_small(const void*, bool, const float*, const float*, const float*, int,
                               int, int64_t, int, int, int32_t*, float*, float*, float*,
                               const float*, float, hipStream_t);
}  // namespace moe

using namespace moe;

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MOE_TRY(expr)                 \
  do {                                \
    int _s = (expr);                  \
    if (_s != MOE_OK) return _s;      \
  } while (0)

// ------------------------------------------------------ kernel timing
// While enabled, each kernel launch is bracketed by two timing events
// recorded on the launch stream (moe_profile_enable / moe_profile_read).
enum KernelId {
  K_ROUTER_LOGITS, K_ROUTER_TOPK, K_AUX_STATS, K_PERMUTE,
  K_FWD_UP, K_FWD_DOWN, K_DGRAD_DOWN, K_DGRAD_UP, K_WGRAD_DOWN, K_WGRAD_UP,
  K_SH_FWD_UP, K_SH_FWD_DOWN, K_SH_DGRAD_DOWN, K_SH_DGRAD_UP, K_SH_WGRAD_DOWN, K_SH_WGRAD_UP,
  K_COMBINE, K_COMBINE_BWD, K_ROUTER_DLOGITS, K_ROUTER_DW, K_ROUTER_DW_REDUCE, K_ROUTER_DX,
  K_UNPERMUTE, K_FILL, K_BIAS_UPDATE, K_QUANT_FP8, K_ROUTER_LOGITS_REDUCE, K_ROUTER_SPLIT, K_COUNT
};
const char* const kKernelNames[K_COUNT] = {
  "router_logits", "router_topk", "aux_stats", "permute",
  "gemm_fwd_up", "gemm_fwd_down", "gemm_dgrad_down", "gemm_dgrad_up", "gemm_wgrad_down",
  "gemm_wgrad_up",
  "gemm_shared_fwd_up", "gemm_shared_fwd_down", "gemm_shared_dgrad_down", "gemm_shared_dgrad_up",
  "gemm_shared_wgrad_down", "gemm_shared_wgrad_up",
  "combine", "combine_bwd", "router_dlogits", "router_dw", "router_dw_reduce", "router_dx",
  "unpermute", "fill_zero", "bias_update", "quant_fp8", "router_logits_reduce", "router_split",
};

struct ProfRec {
  int id;
  hipEvent_t a, b;
};
struct Prof {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t take() {
    std::lock_guard<std::mutex> g(mu);
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Prof& prof() {
  static Prof p;
  return p;
}

class Scope {
 public:
  Scope(int id, hipStream_t s) : id_(id), s_(s) {
    Prof& P = prof();
    if (!P.on.load(std::memory_order_relaxed)) return;
    a_ = P.take();
    b_ = P.take();
    // profiling only: a failed record leaves this launch's time unread
    if (a_ && b_) (void)hipEventRecord(a_, s_);
  }
  ~Scope() {
    if (!a_ || !b_) return;
    (void)hipEventRecord(b_, s_);
    Prof& P = prof();
    std::lock_guard<std::mutex> g(P.mu);
    P.recs.push_back({id_, a_, b_});
  }
 private:
  int id_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
};

constexpr int64_t kMaxE = 1024;
constexpr int64_t kMaxK = 16;

int check_desc(const moe_desc* d) {
  if (!d) return fail(MOE_ERR_INVALID_ARG, "desc is NULL");
  if (d->T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)d->T);
  if (d->E < 1 || d->E > kMaxE)
    return fail(MOE_ERR_INVALID_ARG, "E must be in [1, %lld] (got %lld)", (long long)kMaxE,
                (long long)d->E);
  if (d->k < 1 || d->k > d->E)
    return fail(MOE_ERR_INVALID_ARG, "k must be in [1, E] (got k=%lld, E=%lld)",
                (long long)d->k, (long long)d->E);
  if (d->k > kMaxK)
    return fail(MOE_ERR_UNSUPPORTED, "k > %lld is not supported (got %lld)", (long long)kMaxK,
                (long long)d->k);
  if (d->d < 8 || d->d % 8)
    return fail(MOE_ERR_INVALID_ARG, "d must be a positive multiple of 8 (got %lld)",
                (long long)d->d);
  if (d->f < 8 || d->f % 8)
    return fail(MOE_ERR_INVALID_ARG, "f must be a positive multiple of 8 (got %lld)",
                (long long)d->f);
  if (d->n_shared != 0 && d->n_shared != 1)
    return fail(MOE_ERR_INVALID_ARG, "n_shared must be 0 or 1 (got %lld)", (long long)d->n_shared);
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
  if (!(d->gumbel_tau >= 0.0f) || !std::isfinite(d->gumbel_tau))
    return fail(MOE_ERR_INVALID_ARG, "gumbel_tau must be finite and >= 0");
  if (d->gumbel_tau > 0.0f && d->score != MOE_SOFTMAX)
    return fail(MOE_ERR_UNSUPPORTED, "the noisy gate needs softmax scoring");
  if (d->score != MOE_SOFTMAX && d->score != MOE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "unknown score function %d", d->score);
  if (d->act != MOE_SWIGLU && d->act != MOE_GELU)
    return fail(MOE_ERR_INVALID_ARG, "unknown activation %d", d->act);
  if (d->fp8_grad != MOE_FP8_E4M3 && d->fp8_grad != MOE_FP8_E5M2)
    return fail(MOE_ERR_INVALID_ARG, "unknown FP8 gradient format %d", d->fp8_grad);
  if (d->T * d->k >= (int64_t(1) << 31) || d->T * d->E >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T*k and T*E must be < 2^31");
  {
    // the GEMMs address each operand of one expert through 32-bit byte offsets
    const int64_t es = d->dtype == MOE_BF16 ? 2 : 4;
    const int64_t wid = d->d > 2 * d->f ? d->d : 2 * d->f;
    if (d->T * d->k * wid * es >= (int64_t(1) << 31) || 2 * d->f * d->d * es >= (int64_t(1) << 31))
      return fail(MOE_ERR_UNSUPPORTED, "routed activations or one expert's weights exceed 2 GiB");
  }
  return MOE_OK;
}

int need(const void* p, const char* name) {
  if (!p) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) & 15)
    return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

int opt(const void* p, const char* name) { return p ? need(p, name) : MOE_OK; }

size_t esize(const moe_desc* d) { return d->dtype == MOE_BF16 ? 2 : 4; }
int64_t pre_cols(const moe_desc* d) { return d->act == MOE_SWIGLU ? 2 * d->f : d->f; }
size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Split-K of the router logits (E > 8): enough partitions to give about 512
// workgroups when few 64 x 64 tiles cover T x E, each at least 256 deep.
int route_fwd_splits(const moe_desc* d) {
  if (d->E <= 8) return 1;
  const int64_t tiles = ((d->T + 63) / 64) * ((d->E + 63) / 64);
  int64_t s = (512 + tiles - 1) / tiles;
  const int64_t smax = d->d / 256 > 1 ? d->d / 256 : 1;
  if (s > smax) s = smax;
  if (s > 8) s = 8;
  if (s < 1) s = 1;
  return (int)s;
}

int route_bwd_splits(const moe_desc* d) {
  const int64_t tiles = ((d->E + 63) / 64) * ((d->d + 63) / 64);
  int64_t s = (512 + tiles - 1) / tiles;
  const int64_t smax = d->T / 256 > 1 ? d->T / 256 : 1;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  return (int)s;
}

// Router products of bf16 layers with E > 8 (E a multiple of 8) run on the
// bf16 matrix cores: the float32 operand (W_r forward, the logit gradient
// backward) is split exactly into three bf16 terms and the three products are
// folded in float32. Each GEMM is split into S partitions along K (d forward,
// T backward, each a whole number of 64-deep k-steps) so that its 256 x 256
// tiles cover up to 256 CUs. 0 = not this path.
constexpr int64_t kX3Cus = 256;
// (The GEMM addresses each operand through 32-bit byte offsets: the split
// terms must stay under 2 GiB.)
int router_x3_fwd_splits(const moe_desc* d) {
  if (d->dtype != MOE_BF16 || d->E <= 8 || d->E % 8) return 0;
  if (3 * d->E * d->d * 2 >= (int64_t(1) << 31)) return 0;
  const int64_t tiles = ((d->T + 255) / 256) * ((3 * d->E + 255) / 256);
  for (int s = 4; s > 1; --s)
    if (s * tiles <= kX3Cus && d->d % (64 * s) == 0) return s;
  return 1;
}
// The dense dx_router = dl W_r of the same layers (when the aux or z term
// makes dl dense), both operands float32: one bf16 product over K' = 6E, the
// term pairs (hi, hi), (hi, mid), (mid, hi), (hi, lo), (mid, mid), (lo, hi)
// of dl and W_r laid side by side along K (the pairs dropped are below 2^-24
// of the product). Whether this path applies.
bool router_x3_dense_dx(const moe_desc* d) {
  if (d->dtype != MOE_BF16 || d->E <= 8 || d->E % 8) return false;
  return d->T * 6 * d->E * 2 < (int64_t(1) << 31) && 6 * d->E * d->d * 2 < (int64_t(1) << 31);
}

int router_x3_bwd_splits(const moe_desc* d) {
  if (d->dtype != MOE_BF16 || d->E <= 8 || d->E % 8) return 0;
  if (d->T * 3 * d->E * 2 >= (int64_t(1) << 31)) return 0;
  const int64_t tiles = ((3 * d->E + 255) / 256) * ((d->d + 255) / 256);
  for (int s = 4; s > 1; --s)
    if (s * tiles <= kX3Cus && d->T % (64 * s) == 0) return s;
  return 1;
}

// Split-K of the last, partial round of tiles (bf16 plain-store grouped GEMMs)
// sizes its workspace for at most kTailCusMax CUs per XCD.
constexpr int kTailCusMax = 32;

// CUs per XCD of the current device for the tail split (0 = off: unknown, or
// not eight equal XCDs), capped at kTailCusMax. Cached per device.
int tail_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    cache[dev] = (n > 0 && n % 8 == 0) ? (n / 8 < kTailCusMax ? n / 8 : kTailCusMax) : -1;
  }
  return cache[dev] > 0 ? cache[dev] : 0;
}

// Turn on the tail split for GEMM q with workspace region `tw` (counters cleared).
int enable_tail(GemmArgs& q, void* tw, hipStream_t s) {
  const int c = tail_cus();
  if (c <= 0) return MOE_OK;
  {
    Scope sc(K_FILL, s);
    MOE_TRY(hip_check(launch_fill_zero(tw, tail_counter_bytes(c), s), "clear tail counters"));
  }
  q.tail_ws = tw;
  q.tail_cus = c;
  return MOE_OK;
}

// bytes of the block scales of a rows x K matrix: one byte per 32 elements,
// four to a 32-bit word per 128, words 32-row interleaved (rows padded to a
// multiple of 32)
size_t blk_scale_bytes(int64_t rows, int64_t K) {
  return (size_t)128 * ((K + 127) / 128) * ((rows + 31) / 32);
}

// padded token axis of the FP8 weight gradients' transposed operands: each
// of the E groups starts on a 128-token k-step
int64_t wgrad_rp(const moe_desc* d) { return 128 * ((d->T * d->k + 127) / 128 + d->E); }

// the GEMM addresses block-scale words with 32-bit offsets
bool blk_scale_words_fit(int64_t rows, int64_t K) {
  return blk_scale_bytes(rows, K) / 4 < ((size_t)1 << 31);
}

// The token-axis codes and block scales of the FP8 weight gradients' two
// operands (largest of the two GEMMs; the shared expert's fit in the routed
// ones), the k-step table and two ints of bounds.
size_t wgrad_fp8_ws_bytes(const moe_desc* d) {
  const int64_t Rp = wgrad_rp(d), P = pre_cols(d);
  const int64_t ma = std::max(d->d, P), mb = std::max(d->f, d->d);
  return align256((size_t)ma * Rp) + align256(blk_scale_bytes(ma, Rp)) + align256((size_t)mb * Rp) +
         align256(blk_scale_bytes(mb, Rp)) + align256((size_t)(Rp / 128) * 4) + 256;
}

size_t ws_bytes_for(const moe_desc* d, int op) {
  const int64_t T = d->T, E = d->E;
  switch (op) {
    case MOE_OP_ROUTE: {
      if (const int X = router_x3_fwd_splits(d))
        return align256((size_t)T * E * 4) + align256((size_t)3 * E * d->d * 2) +
               (size_t)X * T * 3 * E * 4;
      const int S = route_fwd_splits(d);
      return align256((size_t)T * E * 4) + (S > 1 ? (size_t)S * T * E * 4 : 0);
    }
    case MOE_OP_AUX_STATS: {
      const size_t nb = (size_t)(T + 255) / 256;
      return align256(nb * E * 8) + align256(nb * E * 4) + align256(nb * 8);
    }
    case MOE_OP_PERMUTE: return align256(perm_ws_bytes((int)T, (int)E));
    case MOE_OP_FFN_FWD: return d->dtype == MOE_BF16 ? tail_ws_bytes(kTailCusMax) : 0;
    case MOE_OP_FFN_BWD:
      return align256((size_t)T * d->k * pre_cols(d) * esize(d)) +
             (d->n_shared ? align256((size_t)T * pre_cols(d) * esize(d)) : 0) +
             (d->dtype == MOE_BF16 ? tail_ws_bytes(kTailCusMax) : 0);
    case MOE_OP_ROUTE_BWD: {
      if (E <= 8) return align256((size_t)router_dw_small_chunks((int)T) * E * d->d * 4);
      if (const int X = router_x3_bwd_splits(d)) {
        // dW_r's split and partial products; the dense dx_router's two
        // operands reuse the region afterwards
        const size_t dw = align256((size_t)T * 3 * E * 2) + (size_t)X * 3 * E * d->d * 4;
        const size_t dx = router_x3_dense_dx(d)
                              ? align256((size_t)T * 6 * E * 2) + (size_t)6 * E * d->d * 2 : 0;
        return dw > dx ? dw : dx;
      }
      const int S = route_bwd_splits(d);
      return S > 1 ? align256((size_t)S * E * d->d * 4) : 0;
    }
    case MOE_OP_FFN_FWD_FP8: {
      // FP8 codes and scale exponents of H between the two GEMMs, then the
      // down-projection's split-K tail
      size_t b = align256((size_t)T * d->k * d->f) + align256((size_t)T * d->k * 4);
      if (d->n_shared) b += align256((size_t)T * d->f) + align256((size_t)T * 4);
      return b + tail_ws_bytes(kTailCusMax);
    }
    case MOE_OP_FFN_BWD_FP8:
    case MOE_OP_FFN_BWD_FP8B: {
      // the bf16 backward's pre-activation gradients, then FP8 codes and
      // scales (an int32 per row, or block scales) of the upstream gradient
      // and of the pre-activation gradient (routed rows; the shared expert's
      // T rows reuse them afterwards)
      const int64_t R = T * d->k, P = pre_cols(d);
      const bool blk = op == MOE_OP_FFN_BWD_FP8B;
      return ws_bytes_for(d, MOE_OP_FFN_BWD) + align256((size_t)R * d->d) +
             align256(blk ? blk_scale_bytes(R, d->d) : (size_t)R * 4) + align256((size_t)R * P) +
             align256(blk ? blk_scale_bytes(R, P) : (size_t)R * 4);
    }
    case MOE_OP_FFN_BWD_FP8W:
      // the FP8 backward's buffers, then the weight gradients' token-axis ones
      return ws_bytes_for(d, MOE_OP_FFN_BWD_FP8) + wgrad_fp8_ws_bytes(d);
    case MOE_OP_FFN_BWD_FP8BW: {
      // the same on the block-scaled backward, plus dO's token-axis codes and
      // scales: they are written with its row blocks before dH and kept for dW2
      const int64_t Rp = wgrad_rp(d);
      return ws_bytes_for(d, MOE_OP_FFN_BWD_FP8B) + wgrad_fp8_ws_bytes(d) + align256((size_t)d->d * Rp) +
             align256(blk_scale_bytes(d->d, Rp));
    }
    case MOE_OP_FFN_FWD_FP8B: {
      // FP8 codes and block scales of H between the two GEMMs, then the
      // down-projection's split-K tail
      size_t b = align256((size_t)T * d->k * d->f) + align256(blk_scale_bytes(T * d->k, d->f));
      if (d->n_shared) b += align256((size_t)T * d->f) + align256(blk_scale_bytes(T, d->f));
      return b + tail_ws_bytes(kTailCusMax);
    }
  }
  return 0;
}

int check_ws(const moe_desc* d, int op, const void* ws, size_t bytes) {
  const size_t want = ws_bytes_for(d, op);
  if (bytes < want)
    return fail(MOE_ERR_WORKSPACE, "workspace too small: need %zu bytes, got %zu", want, bytes);
  if (want && !ws) return fail(MOE_ERR_INVALID_ARG, "ws is NULL");
  if (ws && (reinterpret_cast<uintptr_t>(ws) & 255))
    return fail(MOE_ERR_INVALID_ARG, "ws is not 256-byte aligned");
  return MOE_OK;
}

Operand opnd(const void* base, int64_t ld, int64_t gstride, int rowidx) {
  Operand o;
  o.base = base;
  o.ld = ld;
  o.gstride = gstride;
  o.rowidx = rowidx;
  return o;
}

GemmArgs blank() {
  GemmArgs p;
  memset(&p, 0, sizeof p);
  p.k_splits = 1;
  return p;
}

int run_gemm(const moe_desc* d, const GemmArgs& p, bool akm, bool bkm, int epi, int rag,
             hipStream_t s, const char* what, int kid) {
  Scope sc(kid, s);
  hipError_t e = d->dtype == MOE_BF16 ? gemm_bf16(p, akm, bkm, epi, rag, s)
                                      : gemm_f32(p, akm, bkm, epi, rag, s);
  return hip_check(e, what);
}

// ------------------------------------------------ library-owned scratch
// moe_permute_noalloc keeps the permute's per-block base counts in this
// array instead of a caller workspace. One copy per GPU (each device holds
// its own at its own address); host code never passes the symbol itself to
// a kernel, only the device address hipGetSymbolAddress returns for the
// current device, looked up once per device.
constexpr size_t kScratchBytes = 131072;   // the permute's largest histogram (32768 ints)
static __device__ __align__(256) int32_t scratch[kScratchBytes / 4];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {nullptr};

// device address of `scratch` on the current device (nullptr + error text on failure)
void* scratch_for_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    fail(MOE_ERR_HIP, "scratch: no current device");
    return nullptr;
  }
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      fail(MOE_ERR_HIP, "scratch: hipGetSymbolAddress: %s", hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

int moe_profile_enable(int on) {
  g_err[0] = 0;
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  for (auto& r : P.recs) {
    P.pool.push_back(r.a);
    P.pool.push_back(r.b);
  }
  P.recs.clear();
  P.on.store(on != 0);
  return MOE_OK;
}

int moe_profile_read(int cap, int* n, const char** names, double* total_ms, int* launches) {
  g_err[0] = 0;
  if (!n || cap < 0 || (cap > 0 && (!names || !total_ms || !launches)))
    return fail(MOE_ERR_INVALID_ARG, "bad output arrays");
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  double tot[K_COUNT] = {0};
  int cnt[K_COUNT] = {0};
  int order[K_COUNT];
  int nk = 0;
  for (auto& r : P.recs) {
    hipError_t e = hipEventSynchronize(r.b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_check(e, "profile read");
    if (cnt[r.id] == 0) order[nk++] = r.id;
    tot[r.id] += ms;
    cnt[r.id] += 1;
  }
  for (auto& r : P.recs) {
    P.pool.push_back(r.a);
    P.pool.push_back(r.b);
  }
  P.recs.clear();
  *n = nk;
  for (int i = 0; i < nk && i < cap; ++i) {
    names[i] = kKernelNames[order[i]];
    total_ms[i] = tot[order[i]];
    launches[i] = cnt[order[i]];
  }
  return MOE_OK;
}

const char* moe_last_error(void) { return g_err; }

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

int moe_workspace_size(const moe_desc* desc, int op, size_t* bytes) {
  g_err[0] = 0;
  MOE_TRY(check_desc(desc));
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  if (op < MOE_OP_ROUTE || op > MOE_OP_FFN_BWD_FP8BW)
    return fail(MOE_ERR_INVALID_ARG, "unknown op %d", op);
  *bytes = ws_bytes_for(desc, op);
  return MOE_OK;
}

int moe_capacity(int64_t T, int64_t k, int64_t E, double cf, int64_t* capacity) {
  g_err[0] = 0;
  if (!capacity) return fail(MOE_ERR_INVALID_ARG, "capacity is NULL");
  if (T < 0 || k < 1 || E < 1) return fail(MOE_ERR_INVALID_ARG, "bad T/k/E");
  if (!(cf == cf)) return fail(MOE_ERR_INVALID_ARG, "cf is NaN");
  if (cf < 0) {
    *capacity = -1;
    return MOE_OK;
  }
  const double c = cf * (double)T * (double)k / (double)E;
  *capacity = (int64_t)std::ceil(c);
  return MOE_OK;
}

int moe_route(const moe_desc* desc, const void* x, const float* w_r, const float* logit_bias,
              const float* sel_bias, const float* gumbel_u, int32_t* topk_idx, float* gate,
              float* scores, float* lse, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  MOE_TRY(check_desc(desc));
  MOE_TRY(need(x, "x"));
  MOE_TRY(need(w_r, "w_r"));
  MOE_TRY(opt(logit_bias, "logit_bias"));
  MOE_TRY(opt(sel_bias, "sel_bias"));
  MOE_TRY(need(topk_idx, "topk_idx"));
  MOE_TRY(need(gate, "gate"));
  MOE_TRY(need(scores, "scores"));
  MOE_TRY(opt(lse, "lse"));
  if (desc->gumbel_tau > 0.0f) MOE_TRY(need(gumbel_u, "gumbel_u"));
  else if (gumbel_u) return fail(MOE_ERR_INVALID_ARG, "gumbel_u given but desc->gumbel_tau is 0");
  MOE_TRY(check_ws(desc, MOE_OP_ROUTE, ws, ws_bytes));
  if (desc->T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  if (desc->E <= 8) {
    // few experts: logits, scores and top-k fused in one streaming pass over x
    Scope sc(K_ROUTER_TOPK, s);
    return hip_check(launch_router_small(x, desc->dtype == MOE_BF16, w_r, logit_bias, sel_bias,
                                         (int)desc->T, (int)desc->E, desc->d, (int)desc->k,
                                         desc->score, topk_idx, gate, scores, lse, gumbel_u,
                                         desc->gumbel_tau, s),
                     "router (fused)");
  }
  float* logits = (float*)ws;
  if (const int X = router_x3_fwd_splits(desc)) {
    // logits = x [hi | mid | lo]^T per K partition on the bf16 matrix cores,
    // then (lo + mid) + hi folded over the partitions in order, + logit_bias
    const int64_t T = desc->T, E = desc->E, d = desc->d, Ks = d / X;
    bf16_t* w3 = (bf16_t*)((char*)ws + align256((size_t)T * E * 4));
    float* part = (float*)((char*)w3 + align256((size_t)3 * E * d * 2));
    {
      Scope sc(K_ROUTER_SPLIT, s);
      MOE_TRY(hip_check(launch_split_bf16x3(w_r, E, d, w3, d, E * d, s), "router weight split"));
    }
    GemmArgs p = blank();
    p.a = opnd(x, d, Ks, 0);
    p.b = opnd(w3, d, Ks, 0);
    p.c = part;
    p.ldc = 3 * E;
    p.c_gstride = T * 3 * E;
    p.G = X;
    p.M = T;
    p.N = 3 * E;
    p.K = Ks;
    {
      Scope sc(K_ROUTER_LOGITS, s);
      MOE_TRY(hip_check(gemm_bf16(p, true, true, EPI_STORE_F32, RAG_NONE, s), "router logits"));
    }
    {
      Scope sc(K_ROUTER_LOGITS_REDUCE, s);
      MOE_TRY(hip_check(launch_fold_bf16x3(part, X, T * 3 * E, E, 3 * E, T, E, logit_bias, logits, s),
                        "router logits fold"));
    }
    Scope sc(K_ROUTER_TOPK, s);
    return hip_check(launch_router_topk(logits, (int)desc->T, (int)desc->E, (int)desc->k,
                                        desc->score, sel_bias, topk_idx, gate, scores, lse, gumbel_u,
                                        desc->gumbel_tau, s),
                     "router top-k");
  }
  // logits = x W_r^T (+ logit_bias); with split-K the partitions land after
  // the logits (partition 0 carries the bias) and are folded in order
  const int S = route_fwd_splits(desc);
  float* part = (float*)((char*)ws + align256((size_t)desc->T * desc->E * 4));
  GemmArgs p = blank();
  p.a = opnd(x, desc->d, 0, 1);
  p.b = opnd(w_r, desc->d, 0, 0);
  p.c = S > 1 ? part : logits;
  p.ldc = desc->E;
  p.G = 1;
  p.M = desc->T;
  p.N = desc->E;
  p.K = desc->d;
  p.col_bias = logit_bias;
  p.k_splits = S;
  {
    Scope sc(K_ROUTER_LOGITS, s);
    MOE_TRY(hip_check(gemm_router_logits(p, desc->dtype == MOE_BF16, s), "router logits"));
  }
  if (S > 1) {
    Scope sc(K_ROUTER_LOGITS_REDUCE, s);
    MOE_TRY(hip_check(launch_splitk_reduce(part, S, desc->T * desc->E, logits, s),
                      "router logits reduce"));
  }
  Scope sc(K_ROUTER_TOPK, s);
  return hip_check(launch_router_topk(logits, (int)desc->T, (int)desc->E, (int)desc->k,
                                      desc->score, sel_bias, topk_idx, gate, scores, lse, gumbel_u,
                                      desc->gumbel_tau, s),
                   "router top-k");
}

int moe_aux_stats(const moe_desc* desc, const float* scores, const int32_t* topk_idx,
                  const float* lse, int32_t* counts, float* y, float* z, float* out3, void* ws,
                  size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  MOE_TRY(check_desc(desc));
  MOE_TRY(need(scores, "scores"));
  MOE_TRY(need(topk_idx, "topk_idx"));
  MOE_TRY(need(counts, "counts"));
  MOE_TRY(need(y, "y"));
  MOE_TRY(need(z, "z"));
  MOE_TRY(opt(lse, "lse"));
  MOE_TRY(need(out3, "out3"));
  MOE_TRY(check_ws(desc, MOE_OP_AUX_STATS, ws, ws_bytes));
  if (desc->T == 0) return MOE_OK;
  const size_t nb = (size_t)(desc->T + 255) / 256;
  double* pz = (double*)ws;
  int32_t* pc = (int32_t*)((char*)ws + align256(nb * desc->E * 8));
  double* pl = (double*)((char*)pc + align256(nb * desc->E * 4));
  Scope sc(K_AUX_STATS, (hipStream_t)stream);
  return hip_check(launch_aux_stats(scores, topk_idx, lse, (int)desc->T, (int)desc->E,
                                    (int)desc->k, pz, pc, pl, counts, y, z, out3,
                                    (hipStream_t)stream),
                   "aux stats");
}

int moe_bias_update(const moe_desc* desc, const int32_t* counts, float gamma, float* bias,
                    void* stream) {
  g_err[0] = 0;
  MOE_TRY(check_desc(desc));
  MOE_TRY(need(counts, "counts"));
  MOE_TRY(need(bias, "bias"));
  if (!std::isfinite(gamma)) return fail(MOE_ERR_INVALID_ARG, "gamma is not finite");
  if (desc->T == 0) return MOE_OK;
  Scope sc(K_BIAS_UPDATE, (hipStream_t)stream);
  return hip_check(launch_bias_update(counts, (int)desc->E, desc->T * desc->k, gamma, bias,
                                      (hipStream_t)stream),
                   "bias update");
}

int moe_permute(const moe_desc* desc, const void* x, const int32_t* topk_idx, int32_t* offsets,
                int32_t* row_of, int32_t* token_of, int32_t* n_dropped, void* x_perm, void* ws,
                size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  MOE_TRY(check_desc(desc));
  MOE_TRY(need(x, "x"));
  MOE_TRY(need(topk_idx, "topk_idx"));
  MOE_TRY(need(offsets, "offsets"));
  MOE_TRY(need(row_of, "row_of"));
  MOE_TRY(need(token_of, "token_of"));
  MOE_TRY(need(n_dropped, "n_dropped"));
  MOE_TRY(need(x_perm, "x_perm"));
  MOE_TRY(check_ws(desc, MOE_OP_PERMUTE, ws, ws_bytes));
  if (desc->T == 0) return MOE_OK;
  Scope sc(K_PERMUTE, (hipStream_t)stream);
  return hip_check(launch_permute(x, desc->dtype == MOE_BF16, topk_idx, (int)desc->T,
                                  (int)desc->E, (int)desc->k, desc->d, desc->capacity,
                                  (int32_t*)ws, offsets, row_of, token_of, n_dropped, x_perm,
                                  (hipStream_t)stream),
                   "permute");
}

int moe_permute_noalloc(const moe_desc* desc, const void* x, const int32_t* topk_idx,
                        int32_t* offsets, int32_t* row_of, int32_t* token_of, int32_t* n_dropped,
                        void* x_perm, void* stream) {
  g_err[0] = 0;
  MOE_TRY(check_desc(desc));
  MOE_TRY(need(x, "x"));
  MOE_TRY(need(topk_idx, "topk_idx"));
  MOE_TRY(need(offsets, "offsets"));
  MOE_TRY(need(row_of, "row_of"));
  MOE_TRY(need(token_of, "token_of"));
  MOE_TRY(need(n_dropped, "n_dropped"));
  MOE_TRY(need(x_perm, "x_perm"));
  const size_t want = ws_bytes_for(desc, MOE_OP_PERMUTE);
  if (want > kScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED, "permute needs %zu bytes of scratch, the library holds %zu",
                want, kScratchBytes);
  if (desc->T == 0) return MOE_OK;
  void* base = scratch_for_current_device();
  if (!base) return MOE_ERR_HIP;
  Scope sc(K_PERMUTE, (hipStream_t)stream);
  return hip_check(launch_permute(x, desc->dtype == MOE_BF16, topk_idx, (int)desc->T,
                                  (int)desc->E, (int)desc->k, desc->d, desc->capacity,
                                  (int32_t*)base, offsets, row_of, token_of, n_dropped, x_perm,
                                  (hipStream_t)stream),
                   "permute (library scratch)");
}

int moe_grouped_ffn_fwd(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                        const void* x, const void* w13, const void* w2, const void* sw13,
                        const void* sw2, void* save_pre, void* save_h, void* save_pre_s,
                        void* save_h_s, void* out, void* out_shared, void* ws, size_t ws_bytes,
                        void* stream) {
  g_err[0] = 0;
  MOE_TRY(check_desc(desc));
  MOE_TRY(need(x_perm, "x_perm"));
  MOE_TRY(need(offsets, "offsets"));
  MOE_TRY(need(w13, "w13"));
  MOE_TRY(need(w2, "w2"));
  MOE_TRY(need(save_pre, "save_pre"));
  MOE_TRY(need(save_h, "save_h"));
  MOE_TRY(need(out, "out"));
  if (desc->n_shared) {
    MOE_TRY(need(x, "x"));
    MOE_TRY(need(sw13, "sw13"));
    MOE_TRY(need(sw2, "sw2"));
    MOE_TRY(need(save_pre_s, "save_pre_s"));
    MOE_TRY(need(save_h_s, "save_h_s"));
    MOE_TRY(need(out_shared, "out_shared"));
  }
  MOE_TRY(check_ws(desc, MOE_OP_FFN_FWD, ws, ws_bytes));
  if (desc->T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  const int64_t d = desc->d, f = desc->f, P = pre_cols(desc);
  const int epi1 = desc->act == MOE_SWIGLU ? EPI_SWIGLU_FWD : EPI_GELU_FWD;
  for (int shared = 0; shared <= (int)desc->n_shared; ++shared) {
    const int rag = shared ? RAG_NONE : RAG_M;
    GemmArgs p = blank();
    p.a = opnd(shared ? x : x_perm, d, 0, 1);
    p.b = opnd(shared ? sw13 : w13, d, P * d, 0);
    p.c = shared ? save_h_s : save_h;
    p.ldc = f;
    p.c_rowidx = 1;
    p.aux = shared ? save_pre_s : save_pre;
    p.ldaux = P;
    p.aux_rowidx = 1;
    p.offsets = offsets;
    p.G = shared ? 1 : (int)desc->E;
    p.M = desc->T;
    p.N = f;
    p.K = d;
    p.fdim = f;
    p.max_rows = desc->T * desc->k;
    MOE_TRY(run_gemm(desc, p, true, true, epi1, rag, s, "ffn fwd first matrix",
                     shared ? K_SH_FWD_UP : K_FWD_UP));
    GemmArgs q = blank();
    q.a = opnd(shared ? save_h_s : save_h, f, 0, 1);
    q.b = opnd(shared ? sw2 : w2, f, d * f, 0);
    q.c = shared ? out_shared : out;
    q.ldc = d;
    q.c_rowidx = 1;
    q.offsets = offsets;
    q.G = p.G;
    q.M = desc->T;
    q.N = d;
    q.K = f;
    q.max_rows = p.max_rows;
    if (!shared && desc->dtype == MOE_BF16) MOE_TRY(enable_tail(q, ws, s));
    MOE_TRY(run_gemm(desc, q, true, true, EPI_STORE, rag, s, "ffn fwd down matrix",
                     shared ? K_SH_FWD_DOWN : K_FWD_DOWN));
  }
  return MOE_OK;
}

int moe_quantize_fp8(const void* src, int64_t rows, int64_t K, int64_t ld_src,
                     const int32_t* valid_rows, void* codes, int64_t ld_codes, int32_t* scale_exp,
                     void* stream) {
  g_err[0] = 0;
  if (rows < 0 || rows >= (int64_t(1) << 31))
    return fail(MOE_ERR_INVALID_ARG, "rows must be in [0, 2^31) (got %lld)", (long long)rows);
  if (K < 16 || K % 16)
    return fail(MOE_ERR_INVALID_ARG, "K must be a positive multiple of 16 (got %lld)", (long long)K);
  if (ld_src < K || ld_src % 8)
    return fail(MOE_ERR_INVALID_ARG, "ld_src must be >= K and a multiple of 8 (got %lld)",
                (long long)ld_src);
  if (ld_codes < K || ld_codes % 16)
    return fail(MOE_ERR_INVALID_ARG, "ld_codes must be >= K and a multiple of 16 (got %lld)",
                (long long)ld_codes);
  MOE_TRY(need(src, "src"));
  MOE_TRY(need(codes, "codes"));
  MOE_TRY(need(scale_exp, "scale_exp"));
  if (valid_rows && (reinterpret_cast<uintptr_t>(valid_rows) & 3))
    return fail(MOE_ERR_INVALID_ARG, "valid_rows is not 4-byte aligned");
  if (rows == 0) return MOE_OK;
  Scope sc(K_QUANT_FP8, (hipStream_t)stream);
  return hip_check(launch_quant_fp8(src, rows, K, ld_src, valid_rows, codes, ld_codes, scale_exp,
                                    (hipStream_t)stream),
                   "fp8 quantize");
}

}  // extern "C"

namespace {

// The FP8 forward with per-row exponents (blk = false: int32 per row) or
// block scales (blk = true: bytes, blk_scale_bytes(K) per row).
int ffn_fwd_fp8_impl(bool blk, const moe_desc* desc, const void* xq_perm, const void* sx_perm,
                     const int32_t* offsets, const void* xq, const void* sx, const void* w13q,
                     const void* s13, const void* w2q, const void* s2, const void* sw13q,
                     const void* ss13, const void* sw2q, const void* ss2, void* save_pre,
                     void* save_h, void* save_pre_s, void* save_h_s, void* out, void* out_shared,
                     void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  MOE_TRY(check_desc(desc));
  if (desc->dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "the FP8 forward writes bf16 activations: desc->dtype must be bf16");
  if (desc->d % 16 || desc->f % 16)
    return fail(MOE_ERR_UNSUPPORTED, "the FP8 forward needs d and f multiples of 16");
  MOE_TRY(need(xq_perm, "xq_perm"));
  MOE_TRY(need(sx_perm, "sx_perm"));
  MOE_TRY(need(offsets, "offsets"));
  MOE_TRY(need(w13q, "w13q"));
  MOE_TRY(need(s13, "s13"));
  MOE_TRY(need(w2q, "w2q"));
  MOE_TRY(need(s2, "s2"));
  MOE_TRY(need(save_pre, "save_pre"));
  MOE_TRY(need(save_h, "save_h"));
  MOE_TRY(need(out, "out"));
  if (desc->n_shared) {
    MOE_TRY(need(xq, "xq"));
    MOE_TRY(need(sx, "sx"));
    MOE_TRY(need(sw13q, "sw13q"));
    MOE_TRY(need(ss13, "ss13"));
    MOE_TRY(need(sw2q, "sw2q"));
    MOE_TRY(need(ss2, "ss2"));
    MOE_TRY(need(save_pre_s, "save_pre_s"));
    MOE_TRY(need(save_h_s, "save_h_s"));
    MOE_TRY(need(out_shared, "out_shared"));
  }
  const int op = blk ? MOE_OP_FFN_FWD_FP8B : MOE_OP_FFN_FWD_FP8;
  MOE_TRY(check_ws(desc, op, ws, ws_bytes));
  if (desc->T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  const int64_t T = desc->T, d = desc->d, f = desc->f, P = pre_cols(desc);
  const int epi1 = desc->act == MOE_SWIGLU ? EPI_SWIGLU_FWD : EPI_GELU_FWD;
  if (blk) {
    const int64_t R = T * desc->k;
    if (!blk_scale_words_fit(R, d) || !blk_scale_words_fit(R, f) ||
        !blk_scale_words_fit(desc->E * P, d) || !blk_scale_words_fit(desc->E * d, f))
      return fail(MOE_ERR_UNSUPPORTED, "block scales of this layer exceed 2^31 words");
  }
  // H codes and its scales (an int32 per row, or the block scales) between
  // the GEMMs
  char* w = (char*)ws;
  uint8_t* hq = (uint8_t*)w;
  void* hs = w + align256((size_t)T * desc->k * f);
  uint8_t* hq_s = (uint8_t*)((char*)hs + align256(blk ? blk_scale_bytes(T * desc->k, f)
                                                      : (size_t)T * desc->k * 4));
  void* hs_s = desc->n_shared ? (void*)((char*)hq_s + align256((size_t)T * f)) : nullptr;
  char* tail_w = w + ws_bytes_for(desc, op) - tail_ws_bytes(kTailCusMax);
  for (int shared = 0; shared <= (int)desc->n_shared; ++shared) {
    const int rag = shared ? RAG_NONE : RAG_M;
    GemmArgs p = blank();
    p.a = opnd(shared ? xq : xq_perm, d, 0, 1);
    p.b = opnd(shared ? sw13q : w13q, d, P * d, 0);
    p.a_sexp = (const int32_t*)(shared ? sx : sx_perm);
    p.b_sexp = (const int32_t*)(shared ? ss13 : s13);
    p.b_sexp_gstride = P;
    p.blk_scales = blk;
    p.c = shared ? save_h_s : save_h;
    p.ldc = f;
    p.c_rowidx = 1;
    p.aux = shared ? save_pre_s : save_pre;
    p.ldaux = P;
    p.aux_rowidx = 1;
    p.offsets = offsets;
    p.G = shared ? 1 : (int)desc->E;
    p.M = T;
    p.N = f;
    p.K = d;
    p.fdim = f;
    p.max_rows = T * desc->k;
    {
      Scope sc(shared ? K_SH_FWD_UP : K_FWD_UP, s);
      MOE_TRY(hip_check(gemm_fp8(p, epi1, rag, s), "fp8 ffn fwd first matrix"));
    }
    // H (bf16, kept for the backward) -> FP8 codes for the down-projection;
    // routed rows beyond offsets[E] are skipped on the device
    uint8_t* q8 = shared ? hq_s : hq;
    void* qs = shared ? hs_s : hs;
    {
      Scope sc(K_QUANT_FP8, s);
      const void* hsrc = shared ? save_h_s : save_h;
      const int64_t hrows = shared ? T : T * desc->k;
      const int32_t* hvalid = shared ? nullptr : offsets + desc->E;
      MOE_TRY(hip_check(blk ? launch_quant_fp8_blocks(hsrc, hrows, f, f, hvalid, q8, f, (uint8_t*)qs, s)
                            : launch_quant_fp8(hsrc, hrows, f, f, hvalid, q8, f, (int32_t*)qs, s),
                        "fp8 quantize H"));
    }
    GemmArgs q = blank();
    q.a = opnd(q8, f, 0, 1);
    q.b = opnd(shared ? sw2q : w2q, f, d * f, 0);
    q.a_sexp = (const int32_t*)qs;
    q.b_sexp = (const int32_t*)(shared ? ss2 : s2);
    q.b_sexp_gstride = d;
    q.blk_scales = blk;
    q.c = shared ? out_shared : out;
    q.ldc = d;
    q.c_rowidx = 1;
    q.offsets = offsets;
    q.G = p.G;
    q.M = T;
    q.N = d;
    q.K = f;
    q.max_rows = p.max_rows;
    if (!shared) MOE_TRY(enable_tail(q, tail_w, s));
    Scope sc(shared ? K_SH_FWD_DOWN : K_FWD_DOWN, s);
    MOE_TRY(hip_check(gemm_fp8(q, EPI_STORE, rag, s), "fp8 ffn fwd down matrix"));
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_grouped_ffn_fwd_fp8(const moe_desc* desc, const void* xq_perm, const int32_t* sx_perm,
                            const int32_t* offsets, const void* xq, const int32_t* sx,
                            const void* w13q, const int32_t* s13, const void* w2q,
                            const int32_t* s2, const void* sw13q, const int32_t* ss13,
                            const void* sw2q, const int32_t* ss2, void* save_pre, void* save_h,
                            void* save_pre_s, void* save_h_s, void* out, void* out_shared, void* ws,
                            size_t ws_bytes, void* stream) {
  return ffn_fwd_fp8_impl(false, desc, xq_perm, sx_perm, offsets, xq, sx, w13q, s13, w2q, s2, sw13q,
                          ss13, sw2q, ss2, save_pre, save_h, save_pre_s, save_h_s, out, out_shared, ws,
                          ws_bytes, stream);
}

int moe_grouped_ffn_fwd_fp8b(const moe_desc* desc, const void* xq_perm, const uint8_t* bx_perm,
                             const int32_t* offsets, const void* xq, const uint8_t* bx,
                             const void* w13q, const uint8_t* b13, const void* w2q,
                             const uint8_t* b2, const void* sw13q, const uint8_t* sb13,
                             const void* sw2q, const uint8_t* sb2, void* save_pre, void* save_h,
                             void* save_pre_s, void* save_h_s, void* out, void* out_shared, void* ws,
                             size_t ws_bytes, void* stream) {
  return ffn_fwd_fp8_impl(true, desc, xq_perm, bx_perm, offsets, xq, bx, w13q, b13, w2q, b2, sw13q,
                          sb13, sw2q, sb2, save_pre, save_h, save_pre_s, save_h_s, out, out_shared,
                          ws, ws_bytes, stream);
}

int moe_quantize_fp8_blocks(const void* src, int64_t rows, int64_t K, int64_t ld_src,
                            const int32_t* valid_rows, void* codes, int64_t ld_codes,
                            uint8_t* scales, void* stream) {
  g_err[0] = 0;
  if (rows < 0 || rows >= (int64_t(1) << 31))
    return fail(MOE_ERR_INVALID_ARG, "rows must be in [0, 2^31) (got %lld)", (long long)rows);
  if (K < 16 || K % 16)
    return fail(MOE_ERR_INVALID_ARG, "K must be a positive multiple of 16 (got %lld)", (long long)K);
  if (ld_src < K || ld_src % 8)
    return fail(MOE_ERR_INVALID_ARG, "ld_src must be >= K and a multiple of 8 (got %lld)",
                (long long)ld_src);
  if (ld_codes < K || ld_codes % 16)
    return fail(MOE_ERR_INVALID_ARG, "ld_codes must be >= K and a multiple of 16 (got %lld)",
                (long long)ld_codes);
  MOE_TRY(need(src, "src"));
  MOE_TRY(need(codes, "codes"));
  MOE_TRY(need(scales, "scales"));
  if (valid_rows && (reinterpret_cast<uintptr_t>(valid_rows) & 3))
    return fail(MOE_ERR_INVALID_ARG, "valid_rows is not 4-byte aligned");
  if (!blk_scale_words_fit(rows, K))
    return fail(MOE_ERR_INVALID_ARG, "block scales of %lld x %lld exceed 2^31 words", (long long)rows,
                (long long)K);
  if (rows == 0) return MOE_OK;
  Scope sc(K_QUANT_FP8, (hipStream_t)stream);
  return hip_check(launch_quant_fp8_blocks(src, rows, K, ld_src, valid_rows, codes, ld_codes, scales,
                                           (hipStream_t)stream),
                   "fp8 quantize blocks");
}

int moe_grouped_ffn_bwd(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                        const void* x, const void* w13, const void* w2, const void* sw13,
                        const void* sw2, const void* save_pre, const void* save_h,
                        const void* save_pre_s, const void* save_h_s, const void* dout,
                        const void* dy, void* dx_perm, void* dx_shared, void* dw13, void* dw2,
                        void* dsw13, void* dsw2, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  MOE_TRY(check_desc(desc));
  MOE_TRY(need(x_perm, "x_perm"));
  MOE_TRY(need(offsets, "offsets"));
  MOE_TRY(need(w13, "w13"));
  MOE_TRY(need(w2, "w2"));
  MOE_TRY(need(save_pre, "save_pre"));
  MOE_TRY(need(save_h, "save_h"));
  MOE_TRY(need(dout, "dout"));
  MOE_TRY(need(dx_perm, "dx_perm"));
  MOE_TRY(need(dw13, "dw13"));
  MOE_TRY(need(dw2, "dw2"));
  if (desc->n_shared) {
    MOE_TRY(need(x, "x"));
    MOE_TRY(need(sw13, "sw13"));
    MOE_TRY(need(sw2, "sw2"));
    MOE_TRY(need(save_pre_s, "save_pre_s"));
    MOE_TRY(need(save_h_s, "save_h_s"));
    MOE_TRY(need(dy, "dy"));
    MOE_TRY(need(dx_shared, "dx_shared"));
    MOE_TRY(need(dsw13, "dsw13"));
    MOE_TRY(need(dsw2, "dsw2"));
  }
  MOE_TRY(check_ws(desc, MOE_OP_FFN_BWD, ws, ws_bytes));
  hipStream_t s = (hipStream_t)stream;
  const int64_t d = desc->d, f = desc->f, P = pre_cols(desc);
  if (desc->T == 0) {
    // no rows: every weight gradient is zero
    MOE_TRY(hip_check(launch_fill_zero(dw13, (size_t)desc->E * P * d * esize(desc), s), "zero dw13"));
    MOE_TRY(hip_check(launch_fill_zero(dw2, (size_t)desc->E * d * f * esize(desc), s), "zero dw2"));
    if (desc->n_shared) {
      MOE_TRY(hip_check(launch_fill_zero(dsw13, (size_t)P * d * esize(desc), s), "zero dsw13"));
      MOE_TRY(hip_check(launch_fill_zero(dsw2, (size_t)d * f * esize(desc), s), "zero dsw2"));
    }
    return MOE_OK;
  }
  void* dpre_r = ws;
  void* dpre_s = (char*)ws + align256((size_t)desc->T * desc->k * P * esize(desc));
  // after the dpre regions: the dX GEMM's tail split-K workspace (bf16)
  char* tail_w = (char*)dpre_s + (desc->n_shared ? align256((size_t)desc->T * P * esize(desc)) : 0);
  const int epi_b = desc->act == MOE_SWIGLU ? EPI_SWIGLU_BWD : EPI_GELU_BWD;
  for (int shared = 0; shared <= (int)desc->n_shared; ++shared) {
    const int ragm = shared ? RAG_NONE : RAG_M;
    const int ragk = shared ? RAG_NONE : RAG_K;
    const int G = shared ? 1 : (int)desc->E;
    void* dpre = shared ? dpre_s : dpre_r;
    const void* go = shared ? dy : dout;            // upstream gradient rows
    const void* xin = shared ? x : x_perm;
    const void* hs = shared ? save_h_s : save_h;
    // dgrad 1: dH = dO W2 (W2 read K-strided), activation backward in the epilogue
    GemmArgs p = blank();
    p.a = opnd(go, d, 0, 1);
    p.b = opnd(shared ? sw2 : w2, f, d * f, 0);
    p.c = dpre;
    p.ldc = P;
    p.c_rowidx = 1;
    p.aux = (void*)(shared ? save_pre_s : save_pre);
    p.ldaux = P;
    p.aux_rowidx = 1;
    p.offsets = offsets;
    p.G = G;
    p.M = desc->T;
    p.N = f;
    p.K = d;
    p.fdim = f;
    p.max_rows = desc->T * desc->k;
    MOE_TRY(run_gemm(desc, p, true, false, epi_b, ragm, s, "ffn dgrad down matrix",
                     shared ? K_SH_DGRAD_DOWN : K_DGRAD_DOWN));
    // dgrad 2: dX = dpre W13 (W13 read K-strided)
    GemmArgs q = blank();
    q.a = opnd(dpre, P, 0, 1);
    q.b = opnd(shared ? sw13 : w13, d, P * d, 0);
    q.c = shared ? dx_shared : dx_perm;
    q.ldc = d;
    q.c_rowidx = 1;
    q.offsets = offsets;
    q.G = G;
    q.M = desc->T;
    q.N = d;
    q.K = P;
    q.max_rows = p.max_rows;
    if (!shared && desc->dtype == MOE_BF16) MOE_TRY(enable_tail(q, tail_w, s));
    MOE_TRY(run_gemm(desc, q, true, false, EPI_STORE, ragm, s, "ffn dgrad first matrix",
                     shared ? K_SH_DGRAD_UP : K_DGRAD_UP));
    // wgrad 2: dW2 = dO^T H (reduce over the expert's rows)
    GemmArgs r = blank();
    r.a = opnd(go, d, 0, 1);
    r.b = opnd(hs, f, 0, 1);
    r.c = shared ? dsw2 : dw2;
    r.ldc = f;
    r.c_gstride = d * f;
    r.offsets = offsets;
    r.G = G;
    r.M = d;
    r.N = f;
    r.K = desc->T;
    MOE_TRY(run_gemm(desc, r, false, false, EPI_STORE, ragk, s, "ffn wgrad down matrix",
                     shared ? K_SH_WGRAD_DOWN : K_WGRAD_DOWN));
    // wgrad 1: dW13 = dpre^T X
    GemmArgs w = blank();
    w.a = opnd(dpre, P, 0, 1);
    w.b = opnd(xin, d, 0, 1);
    w.c = shared ? dsw13 : dw13;
    w.ldc = d;
    w.c_gstride = P * d;
    w.offsets = offsets;
    w.G = G;
    w.M = P;
    w.N = d;
    w.K = desc->T;
    MOE_TRY(run_gemm(desc, w, false, false, EPI_STORE, ragk, s, "ffn wgrad first matrix",
                     shared ? K_SH_WGRAD_UP : K_WGRAD_UP));
  }
  return MOE_OK;
}

int moe_quantize_fp8_t(const void* src, int64_t G, int64_t R, int64_t C, void* codes,
                       int32_t* scale_exp, void* stream) {
  g_err[0] = 0;
  if (G < 0 || G > 65535)
    return fail(MOE_ERR_INVALID_ARG, "G must be in [0, 65535] (got %lld)", (long long)G);
  if (R < 16 || R % 16 || R > (int64_t(1) << 22))
    return fail(MOE_ERR_INVALID_ARG, "R must be a positive multiple of 16, at most 2^22 (got %lld)",
                (long long)R);
  if (C < 8 || C % 8 || C >= (int64_t(1) << 31))
    return fail(MOE_ERR_INVALID_ARG, "C must be a positive multiple of 8 below 2^31 (got %lld)",
                (long long)C);
  MOE_TRY(need(src, "src"));
  MOE_TRY(need(codes, "codes"));
  MOE_TRY(need(scale_exp, "scale_exp"));
  if (G == 0) return MOE_OK;
  Scope sc(K_QUANT_FP8, (hipStream_t)stream);
  return hip_check(launch_quant_fp8_t(src, G, R, C, codes, scale_exp, (hipStream_t)stream),
                   "fp8 transposing quantize");
}

int moe_quantize_fp8_squares(const void* src, int64_t G, int64_t R, int64_t C, void* codes,
                             uint8_t* scales, void* codes_t, uint8_t* scales_t, void* stream) {
  g_err[0] = 0;
  if (G < 0 || G > 65535)
    return fail(MOE_ERR_INVALID_ARG, "G must be in [0, 65535] (got %lld)", (long long)G);
  if (R < 16 || R % 16 || R > (int64_t(1) << 22))
    return fail(MOE_ERR_INVALID_ARG, "R must be a positive multiple of 16, at most 2^22 (got %lld)",
                (long long)R);
  if (C < 16 || C % 16 || C > (int64_t(1) << 22))
    return fail(MOE_ERR_INVALID_ARG, "C must be a positive multiple of 16, at most 2^22 (got %lld)",
                (long long)C);
  MOE_TRY(need(src, "src"));
  if (!codes != !scales || !codes_t != !scales_t)
    return fail(MOE_ERR_INVALID_ARG, "codes and scales (and codes_t and scales_t) are given together");
  if (!codes && !codes_t) return fail(MOE_ERR_INVALID_ARG, "codes and codes_t are both NULL");
  MOE_TRY(opt(codes, "codes"));
  MOE_TRY(opt(scales, "scales"));
  MOE_TRY(opt(codes_t, "codes_t"));
  MOE_TRY(opt(scales_t, "scales_t"));
  if (!blk_scale_words_fit(G * R, C) || !blk_scale_words_fit(G * C, R))
    return fail(MOE_ERR_INVALID_ARG, "block scales of %lld matrices of %lld x %lld exceed 2^31 words",
                (long long)G, (long long)R, (long long)C);
  if (G == 0) return MOE_OK;
  Scope sc(K_QUANT_FP8, (hipStream_t)stream);
  return hip_check(launch_quant_fp8_squares(src, G, R, C, codes, scales, codes_t, scales_t,
                                            (hipStream_t)stream),
                   "fp8 quantize squares");
}

int moe_quantize_fp8_both(const void* src, int64_t G, int64_t R, int64_t C, void* codes,
                          int32_t* scale_exp, void* codes_t, int32_t* scale_exp_t, void* ws,
                          size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (G < 0 || G > 65535)
    return fail(MOE_ERR_INVALID_ARG, "G must be in [0, 65535] (got %lld)", (long long)G);
  if (R < 16 || R % 16 || R > (int64_t(1) << 22))
    return fail(MOE_ERR_INVALID_ARG, "R must be a positive multiple of 16, at most 2^22 (got %lld)",
                (long long)R);
  if (C < 16 || C % 16 || C > 32768)
    return fail(MOE_ERR_INVALID_ARG, "C must be a positive multiple of 16, at most 32768 (got %lld)",
                (long long)C);
  MOE_TRY(need(src, "src"));
  MOE_TRY(need(codes, "codes"));
  MOE_TRY(need(scale_exp, "scale_exp"));
  MOE_TRY(need(codes_t, "codes_t"));
  MOE_TRY(need(scale_exp_t, "scale_exp_t"));
  if (G == 0) return MOE_OK;
  const size_t need_ws = quant_fp8_both_ws(G, R, C);
  if (!ws || ws_bytes < need_ws)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need_ws, ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return fail(MOE_ERR_INVALID_ARG, "ws is not 256-byte aligned");
  Scope sc(K_QUANT_FP8, (hipStream_t)stream);
  return hip_check(launch_quant_fp8_both(src, G, R, C, codes, scale_exp, codes_t, scale_exp_t, ws,
                                         (hipStream_t)stream),
                   "fp8 quantize both orientations");
}

}  // extern "C"

namespace {

// The FP8 backward: data gradients on per-row FP8 operands (blk = false:
// s13_t .. ss2_t are int32 exponents) or on block-scaled ones (blk: they are
// the square-block weights' scale bytes), weight gradients in bf16
// (fp8w = false) or on token-axis block-scaled FP8 operands.
int ffn_bwd_fp8_impl(bool blk, bool fp8w, const moe_desc* desc, const void* x_perm,
                     const int32_t* offsets,
                     const void* x, const void* w13q_t, const int32_t* s13_t, const void* w2q_t,
                     const int32_t* s2_t, const void* sw13q_t, const int32_t* ss13_t,
                     const void* sw2q_t, const int32_t* ss2_t, const void* save_pre,
                     const void* save_h, const void* save_pre_s, const void* save_h_s,
                     const void* dout, const void* dy, void* dx_perm, void* dx_shared, void* dw13,
                     void* dw2, void* dsw13, void* dsw2, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  MOE_TRY(check_desc(desc));
  if (desc->dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "the FP8 backward reads bf16 activations: desc->dtype must be bf16");
  if (desc->d % 16 || desc->f % 16)
    return fail(MOE_ERR_UNSUPPORTED, "the FP8 backward needs d and f multiples of 16");
  MOE_TRY(need(x_perm, "x_perm"));
  MOE_TRY(need(offsets, "offsets"));
  MOE_TRY(need(w13q_t, "w13q_t"));
  MOE_TRY(need(s13_t, "s13_t"));
  MOE_TRY(need(w2q_t, "w2q_t"));
  MOE_TRY(need(s2_t, "s2_t"));
  MOE_TRY(need(save_pre, "save_pre"));
  MOE_TRY(need(save_h, "save_h"));
  MOE_TRY(need(dout, "dout"));
  MOE_TRY(need(dx_perm, "dx_perm"));
  MOE_TRY(need(dw13, "dw13"));
  MOE_TRY(need(dw2, "dw2"));
  if (desc->n_shared) {
    MOE_TRY(need(x, "x"));
    MOE_TRY(need(sw13q_t, "sw13q_t"));
    MOE_TRY(need(ss13_t, "ss13_t"));
    MOE_TRY(need(sw2q_t, "sw2q_t"));
    MOE_TRY(need(ss2_t, "ss2_t"));
    MOE_TRY(need(save_pre_s, "save_pre_s"));
    MOE_TRY(need(save_h_s, "save_h_s"));
    MOE_TRY(need(dy, "dy"));
    MOE_TRY(need(dx_shared, "dx_shared"));
    MOE_TRY(need(dsw13, "dsw13"));
    MOE_TRY(need(dsw2, "dsw2"));
  }
  const int op = blk ? (fp8w ? MOE_OP_FFN_BWD_FP8BW : MOE_OP_FFN_BWD_FP8B)
                     : (fp8w ? MOE_OP_FFN_BWD_FP8W : MOE_OP_FFN_BWD_FP8);
  MOE_TRY(check_ws(desc, op, ws, ws_bytes));
  hipStream_t s = (hipStream_t)stream;
  const int64_t T = desc->T, d = desc->d, f = desc->f, P = pre_cols(desc);
  const int64_t Rp = wgrad_rp(desc);
  const int gf = desc->fp8_grad;   // FP8 format of the gradient operands (0 E4M3, 1 E5M2)
  if (fp8w && (std::max(d, P) * Rp >= (int64_t(1) << 31) || std::max(f, d) * Rp >= (int64_t(1) << 31) ||
               !blk_scale_words_fit(std::max(d, P), Rp) || !blk_scale_words_fit(std::max(f, d), Rp)))
    return fail(MOE_ERR_UNSUPPORTED, "FP8 weight gradients: the token-axis codes exceed 2^31 bytes");
  if (blk && (!blk_scale_words_fit(T * desc->k, d) || !blk_scale_words_fit(T * desc->k, P) ||
              !blk_scale_words_fit(desc->E * f, d) || !blk_scale_words_fit(desc->E * d, P)))
    return fail(MOE_ERR_UNSUPPORTED, "block scales of this layer exceed 2^31 words");
  if (T == 0) {
    // no rows: every weight gradient is zero
    MOE_TRY(hip_check(launch_fill_zero(dw13, (size_t)desc->E * P * d * 2, s), "zero dw13"));
    MOE_TRY(hip_check(launch_fill_zero(dw2, (size_t)desc->E * d * f * 2, s), "zero dw2"));
    if (desc->n_shared) {
      MOE_TRY(hip_check(launch_fill_zero(dsw13, (size_t)P * d * 2, s), "zero dsw13"));
      MOE_TRY(hip_check(launch_fill_zero(dsw2, (size_t)d * f * 2, s), "zero dsw2"));
    }
    return MOE_OK;
  }
  // workspace: the bf16 backward's dpre regions, then the FP8 buffers
  char* wb = (char*)ws;
  void* dpre_r = wb;
  void* dpre_s = wb + align256((size_t)T * desc->k * P * 2);
  // the bf16 backward's layout: after the dpre regions, the dX GEMM's split-K tail
  char* tail_w = (char*)dpre_s + (desc->n_shared ? align256((size_t)T * P * 2) : 0);
  char* w8 = wb + ws_bytes_for(desc, MOE_OP_FFN_BWD);
  // codes and scales of dO and dpre: an int32 exponent per row, or block
  // scale bytes (blk)
  const int64_t RK = T * desc->k;
  uint8_t* gq = (uint8_t*)w8;
  int32_t* gs = (int32_t*)(w8 + align256((size_t)RK * d));
  uint8_t* pq = (uint8_t*)((char*)gs + align256(blk ? blk_scale_bytes(RK, d) : (size_t)RK * 4));
  int32_t* ps = (int32_t*)((char*)pq + align256((size_t)RK * P));
  // FP8 weight gradients: token-axis codes and scales of the two operands,
  // the k-step -> group table and the shared expert's one-group bounds
  char* w9 = w8 + (ws_bytes_for(desc, blk ? MOE_OP_FFN_BWD_FP8B : MOE_OP_FFN_BWD_FP8) -
                   ws_bytes_for(desc, MOE_OP_FFN_BWD));
  uint8_t* qa = (uint8_t*)w9;
  uint8_t* qa_s = qa + align256((size_t)std::max(d, P) * Rp);
  uint8_t* qb = qa_s + align256(blk_scale_bytes(std::max(d, P), Rp));
  uint8_t* qb_s = qb + align256((size_t)std::max(f, d) * Rp);
  int32_t* ktab = (int32_t*)(qb_s + align256(blk_scale_bytes(std::max(f, d), Rp)));
  int32_t* bounds = (int32_t*)((char*)ktab + align256((size_t)(Rp / 128) * 4));
  // block scales with FP8 weight gradients: dO and dpre are each read once
  // for both their row blocks (the data gradients) and their token-axis
  // blocks (the weight gradients); dO's token-axis codes wait in qd for dW2
  const bool fuse = blk && fp8w;
  uint8_t* qd = fuse ? (uint8_t*)w9 + wgrad_fp8_ws_bytes(desc) : nullptr;
  uint8_t* qd_s = fuse ? qd + align256((size_t)d * Rp) : nullptr;
  const int epi_b = desc->act == MOE_SWIGLU ? EPI_SWIGLU_BWD : EPI_GELU_BWD;
  for (int shared = 0; shared <= (int)desc->n_shared; ++shared) {
    const int ragm = shared ? RAG_NONE : RAG_M;
    const int ragk = shared ? RAG_NONE : RAG_K;
    const int G = shared ? 1 : (int)desc->E;
    const int64_t rows = shared ? T : T * desc->k;
    const int32_t* valid = shared ? nullptr : offsets + desc->E;
    void* dpre = shared ? dpre_s : dpre_r;
    const void* go = shared ? dy : dout;            // upstream gradient rows
    const void* xin = shared ? x : x_perm;
    const void* hs = shared ? save_h_s : save_h;
    // group bounds of the token-axis quantizers (the shared expert: one group)
    const int32_t* off = offsets;
    if (fp8w && shared) {
      MOE_TRY(hip_check(launch_set_bounds(bounds, 0, (int32_t)T, s), "shared bounds"));
      off = bounds;
    }
    // upstream gradient -> FP8 rows (routed rows beyond offsets[E] skipped)
    {
      Scope sc(K_QUANT_FP8, s);
      if (fuse)
        MOE_TRY(hip_check(launch_quant_fp8_tblocks(go, rows, d, off, G, ktab, qd, qd_s, s, gf, gq, (uint8_t*)gs),
                          "fp8 quantize dO (rows and token axis)"));
      else
        MOE_TRY(hip_check(blk ? launch_quant_fp8_blocks(go, rows, d, d, valid, gq, d, (uint8_t*)gs, s, gf)
                              : launch_quant_fp8(go, rows, d, d, valid, gq, d, gs, s, gf),
                          "fp8 quantize dO"));
    }
    // dgrad 1: dH = dO W2 against W2^T in FP8, activation backward in the epilogue
    GemmArgs p = blank();
    p.a = opnd(gq, d, 0, 1);
    p.b = opnd(shared ? sw2q_t : w2q_t, d, f * d, 0);
    p.a_sexp = gs;
    p.b_sexp = shared ? ss2_t : s2_t;
    p.b_sexp_gstride = f;
    p.blk_scales = blk;
    p.c = dpre;
    p.ldc = P;
    p.c_rowidx = 1;
    p.aux = (void*)(shared ? save_pre_s : save_pre);
    p.ldaux = P;
    p.aux_rowidx = 1;
    p.offsets = offsets;
    p.G = G;
    p.M = T;
    p.N = f;
    p.K = d;
    p.fdim = f;
    p.max_rows = T * desc->k;
    {
      Scope sc(shared ? K_SH_DGRAD_DOWN : K_DGRAD_DOWN, s);
      MOE_TRY(hip_check(gemm_fp8(p, epi_b, ragm, s, gf), "fp8 ffn dgrad down matrix"));
    }
    // the bf16 pre-activation gradient -> FP8 rows
    {
      Scope sc(K_QUANT_FP8, s);
      if (fuse)
        MOE_TRY(hip_check(launch_quant_fp8_tblocks(dpre, rows, P, off, G, ktab, qa, qa_s, s, gf, pq, (uint8_t*)ps),
                          "fp8 quantize dpre (rows and token axis)"));
      else
        MOE_TRY(hip_check(blk ? launch_quant_fp8_blocks(dpre, rows, P, P, valid, pq, P, (uint8_t*)ps, s, gf)
                              : launch_quant_fp8(dpre, rows, P, P, valid, pq, P, ps, s, gf),
                          "fp8 quantize dpre"));
    }
    // dgrad 2: dX = dpre W13 against W13^T in FP8
    GemmArgs q = blank();
    q.a = opnd(pq, P, 0, 1);
    q.b = opnd(shared ? sw13q_t : w13q_t, P, d * P, 0);
    q.a_sexp = ps;
    q.b_sexp = shared ? ss13_t : s13_t;
    q.b_sexp_gstride = d;
    q.blk_scales = blk;
    q.c = shared ? dx_shared : dx_perm;
    q.ldc = d;
    q.c_rowidx = 1;
    q.offsets = offsets;
    q.G = G;
    q.M = T;
    q.N = d;
    q.K = P;
    q.max_rows = p.max_rows;
    if (!shared) MOE_TRY(enable_tail(q, tail_w, s));
    {
      Scope sc(shared ? K_SH_DGRAD_UP : K_DGRAD_UP, s);
      MOE_TRY(hip_check(gemm_fp8(q, EPI_STORE, ragm, s, gf), "fp8 ffn dgrad first matrix"));
    }
    if (fp8w) {
      // weight gradients on token-axis FP8 operands (block scales per 32 of
      // each expert's tokens): dW2 = dO^T H, then dW13 = dpre^T X
      const int64_t R = rows;
      const int64_t rp = 128 * ((R + 127) / 128 + G);
      auto quant_t = [&](const void* src, int64_t C, uint8_t* codes, uint8_t* sc, int fmt) {
        Scope q(K_QUANT_FP8, s);
        return hip_check(launch_quant_fp8_tblocks(src, R, C, off, G, ktab, codes, sc, s, fmt),
                         "fp8 token-axis quantize");
      };
      for (int which = 0; which < 2; ++which) {
        const bool down = which == 0;
        const int64_t M = down ? d : P, N = down ? f : d;
        // the gradient operand (already quantized with its row blocks when fused)
        if (!fuse) MOE_TRY(quant_t(down ? go : dpre, M, qa, qa_s, gf));
        MOE_TRY(quant_t(down ? hs : xin, N, qb, qb_s, 0));
        const bool kept = fuse && down;   // dO's token-axis codes in qd
        GemmArgs r = blank();
        r.a = opnd(kept ? qd : qa, rp, 0, 0);
        r.b = opnd(qb, rp, 0, 0);
        r.a_sexp = (const int32_t*)(kept ? qd_s : qa_s);
        r.b_sexp = (const int32_t*)qb_s;
        r.b_sexp_gstride = 0;
        r.blk_scales = 1;
        r.c = down ? (shared ? dsw2 : dw2) : (shared ? dsw13 : dw13);
        r.ldc = N;
        r.c_gstride = M * N;
        r.offsets = off;
        r.G = G;
        r.M = M;
        r.N = N;
        r.K = R;
        Scope sc(down ? (shared ? K_SH_WGRAD_DOWN : K_WGRAD_DOWN) : (shared ? K_SH_WGRAD_UP : K_WGRAD_UP), s);
        MOE_TRY(hip_check(gemm_fp8(r, EPI_STORE, RAG_K, s, gf),
                          down ? "fp8 ffn wgrad down matrix" : "fp8 ffn wgrad first matrix"));
      }
      continue;
    }
    // weight gradients in bf16, as in moe_grouped_ffn_bwd
    GemmArgs r = blank();
    r.a = opnd(go, d, 0, 1);
    r.b = opnd(hs, f, 0, 1);
    r.c = shared ? dsw2 : dw2;
    r.ldc = f;
    r.c_gstride = d * f;
    r.offsets = offsets;
    r.G = G;
    r.M = d;
    r.N = f;
    r.K = T;
    MOE_TRY(run_gemm(desc, r, false, false, EPI_STORE, ragk, s, "ffn wgrad down matrix",
                     shared ? K_SH_WGRAD_DOWN : K_WGRAD_DOWN));
    GemmArgs w = blank();
    w.a = opnd(dpre, P, 0, 1);
    w.b = opnd(xin, d, 0, 1);
    w.c = shared ? dsw13 : dw13;
    w.ldc = d;
    w.c_gstride = P * d;
    w.offsets = offsets;
    w.G = G;
    w.M = P;
    w.N = d;
    w.K = T;
    MOE_TRY(run_gemm(desc, w, false, false, EPI_STORE, ragk, s, "ffn wgrad first matrix",
                     shared ? K_SH_WGRAD_UP : K_WGRAD_UP));
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_grouped_ffn_bwd_fp8(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                            const void* x, const void* w13q_t, const int32_t* s13_t,
                            const void* w2q_t, const int32_t* s2_t, const void* sw13q_t,
                            const int32_t* ss13_t, const void* sw2q_t, const int32_t* ss2_t,
                            const void* save_pre, const void* save_h, const void* save_pre_s,
                            const void* save_h_s, const void* dout, const void* dy, void* dx_perm,
                            void* dx_shared, void* dw13, void* dw2, void* dsw13, void* dsw2,
                            void* ws, size_t ws_bytes, void* stream) {
  return ffn_bwd_fp8_impl(false, false, desc, x_perm, offsets, x, w13q_t, s13_t, w2q_t, s2_t, sw13q_t,
                          ss13_t, sw2q_t, ss2_t, save_pre, save_h, save_pre_s, save_h_s, dout, dy,
                          dx_perm, dx_shared, dw13, dw2, dsw13, dsw2, ws, ws_bytes, stream);
}

int moe_grouped_ffn_bwd_fp8w(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                             const void* x, const void* w13q_t, const int32_t* s13_t,
                             const void* w2q_t, const int32_t* s2_t, const void* sw13q_t,
                             const int32_t* ss13_t, const void* sw2q_t, const int32_t* ss2_t,
                             const void* save_pre, const void* save_h, const void* save_pre_s,
                             const void* save_h_s, const void* dout, const void* dy, void* dx_perm,
                             void* dx_shared, void* dw13, void* dw2, void* dsw13, void* dsw2,
                             void* ws, size_t ws_bytes, void* stream) {
  return ffn_bwd_fp8_impl(false, true, desc, x_perm, offsets, x, w13q_t, s13_t, w2q_t, s2_t, sw13q_t,
                          ss13_t, sw2q_t, ss2_t, save_pre, save_h, save_pre_s, save_h_s, dout, dy,
                          dx_perm, dx_shared, dw13, dw2, dsw13, dsw2, ws, ws_bytes, stream);
}

int moe_grouped_ffn_bwd_fp8b(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                             const void* x, const void* w13q_t, const uint8_t* b13_t,
                             const void* w2q_t, const uint8_t* b2_t, const void* sw13q_t,
                             const uint8_t* sb13_t, const void* sw2q_t, const uint8_t* sb2_t,
                             const void* save_pre, const void* save_h, const void* save_pre_s,
                             const void* save_h_s, const void* dout, const void* dy, void* dx_perm,
                             void* dx_shared, void* dw13, void* dw2, void* dsw13, void* dsw2,
                             void* ws, size_t ws_bytes, void* stream) {
  return ffn_bwd_fp8_impl(true, false, desc, x_perm, offsets, x, w13q_t, (const int32_t*)b13_t, w2q_t,
                          (const int32_t*)b2_t, sw13q_t, (const int32_t*)sb13_t, sw2q_t,
                          (const int32_t*)sb2_t, save_pre, save_h, save_pre_s, save_h_s, dout, dy,
                          dx_perm, dx_shared, dw13, dw2, dsw13, dsw2, ws, ws_bytes, stream);
}

int moe_grouped_ffn_bwd_fp8bw(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                              const void* x, const void* w13q_t, const uint8_t* b13_t,
                              const void* w2q_t, const uint8_t* b2_t, const void* sw13q_t,
                              const uint8_t* sb13_t, const void* sw2q_t, const uint8_t* sb2_t,
                              const void* save_pre, const void* save_h, const void* save_pre_s,
                              const void* save_h_s, const void* dout, const void* dy, void* dx_perm,
                              void* dx_shared, void* dw13, void* dw2, void* dsw13, void* dsw2,
                              void* ws, size_t ws_bytes, void* stream) {
  return ffn_bwd_fp8_impl(true, true, desc, x_perm, offsets, x, w13q_t, (const int32_t*)b13_t, w2q_t,
                          (const int32_t*)b2_t, sw13q_t, (const int32_t*)sb13_t, sw2q_t,
                          (const int32_t*)sb2_t, save_pre, save_h, save_pre_s, save_h_s, dout, dy,
                          dx_perm, dx_shared, dw13, dw2, dsw13, dsw2, ws, ws_bytes, stream);
}

int moe_combine(const moe_desc* desc, const void* out, const void* out_shared, const float* gate,
                const int32_t* row_of, void* y, void* stream) {
  g_err[0] = 0;
  MOE_TRY(check_desc(desc));
  MOE_TRY(need(out, "out"));
  MOE_TRY(opt(out_shared, "out_shared"));
  MOE_TRY(need(gate, "gate"));
  MOE_TRY(need(row_of, "row_of"));
  MOE_TRY(need(y, "y"));
  if (desc->T == 0) return MOE_OK;
  Scope sc(K_COMBINE, (hipStream_t)stream);
  return hip_check(launch_combine(out, out_shared, desc->dtype == MOE_BF16, gate, row_of,
                                  (int)desc->T, (int)desc->k, desc->d, y, (hipStream_t)stream),
                   "combine");
}

int moe_combine_bwd(const moe_desc* desc, const void* dy, const void* out, const float* gate,
                    const int32_t* row_of, float* dgate, void* dout, void* stream) {
  g_err[0] = 0;
  MOE_TRY(check_desc(desc));
  MOE_TRY(need(dy, "dy"));
  MOE_TRY(need(out, "out"));
  MOE_TRY(need(gate, "gate"));
  MOE_TRY(need(row_of, "row_of"));
  MOE_TRY(need(dgate, "dgate"));
  MOE_TRY(need(dout, "dout"));
  if (desc->T == 0) return MOE_OK;
  Scope sc(K_COMBINE_BWD, (hipStream_t)stream);
  return hip_check(launch_combine_bwd(dy, out, desc->dtype == MOE_BF16, gate, row_of,
                                      (int)desc->T, (int)desc->k, desc->d, dgate, dout,
                                      (hipStream_t)stream),
                   "combine bwd");
}

int moe_route_bwd(const moe_desc* desc, const void* x, const float* w_r, const float* scores,
                  const int32_t* topk_idx, const float* gate, const float* dgate, const float* y,
                  float aux_coef, const float* lse, float z_coef, float* dlogits,
                  float* dx_router, float* dw_r, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  MOE_TRY(check_desc(desc));
  MOE_TRY(need(x, "x"));
  MOE_TRY(need(w_r, "w_r"));
  MOE_TRY(need(scores, "scores"));
  MOE_TRY(need(topk_idx, "topk_idx"));
  MOE_TRY(need(gate, "gate"));
  MOE_TRY(need(dgate, "dgate"));
  if (aux_coef != 0.0f) MOE_TRY(need(y, "y"));
  if (!(aux_coef == aux_coef)) return fail(MOE_ERR_INVALID_ARG, "aux_coef is NaN");
  if (!(z_coef == z_coef)) return fail(MOE_ERR_INVALID_ARG, "z_coef is NaN");
  if (z_coef != 0.0f) {
    if (desc->score != MOE_SOFTMAX)
      return fail(MOE_ERR_UNSUPPORTED, "z-loss gradient needs softmax scoring");
    MOE_TRY(need(lse, "lse"));
  }
  MOE_TRY(need(dlogits, "dlogits"));
  MOE_TRY(need(dx_router, "dx_router"));
  MOE_TRY(need(dw_r, "dw_r"));
  MOE_TRY(check_ws(desc, MOE_OP_ROUTE_BWD, ws, ws_bytes));
  hipStream_t s = (hipStream_t)stream;
  if (desc->T == 0)
    return hip_check(launch_fill_zero(dw_r, (size_t)desc->E * desc->d * 4, s), "zero dw_r");
  const int T = (int)desc->T, E = (int)desc->E, k = (int)desc->k;
  {
    Scope sc(K_ROUTER_DLOGITS, s);
    const float inv_tau = desc->gumbel_tau > 0.0f ? 1.0f / desc->gumbel_tau : 1.0f;
    MOE_TRY(hip_check(launch_router_dlogits(scores, topk_idx, gate, dgate, y, aux_coef, lse,
                                            z_coef, inv_tau, T, E, k, desc->score, dlogits, s),
                      "router dlogits"));
  }
  if (E <= 8) {
    // few experts: one streaming pass over x, 64-token partials folded in order
    const int S = router_dw_small_chunks(T);
    {
      Scope sc(K_ROUTER_DW, s);
      MOE_TRY(hip_check(launch_router_dw_small(dlogits, x, desc->dtype == MOE_BF16, T, E, desc->d,
                                               (float*)ws, s),
                        "router dw"));
    }
    {
      Scope sc(K_ROUTER_DW_REDUCE, s);
      MOE_TRY(hip_check(launch_splitk_reduce((const float*)ws, S, (int64_t)E * desc->d, dw_r, s),
                        "router dw reduce"));
    }
  } else if (const int X = router_x3_bwd_splits(desc)) {
    // dw_r = [hi | mid | lo]^T x of the split logit gradient per token
    // partition on the bf16 matrix cores, (lo + mid) + hi folded in order
    const int64_t d = desc->d, Ts = (int64_t)T / X;
    bf16_t* dl3 = (bf16_t*)ws;
    float* part = (float*)((char*)ws + align256((size_t)T * 3 * E * 2));
    {
      Scope sc(K_ROUTER_SPLIT, s);
      MOE_TRY(hip_check(launch_split_bf16x3(dlogits, T, E, dl3, 3 * E, E, s), "router dlogits split"));
    }
    GemmArgs p = blank();
    p.a = opnd(dl3, 3 * E, Ts * 3 * E, 0);
    p.b = opnd(x, d, Ts * d, 0);
    p.c = part;
    p.ldc = d;
    p.c_gstride = 3 * E * d;
    p.G = X;
    p.M = 3 * E;
    p.N = d;
    p.K = Ts;
    {
      Scope sc(K_ROUTER_DW, s);
      MOE_TRY(hip_check(gemm_bf16(p, false, false, EPI_STORE_F32, RAG_NONE, s), "router dw"));
    }
    {
      Scope sc(K_ROUTER_DW_REDUCE, s);
      MOE_TRY(hip_check(launch_fold_bf16x3(part, X, 3 * E * d, E * d, d, E, d, nullptr, dw_r, s),
                        "router dw fold"));
    }
  } else {
  // dw_r = dl^T x, split over tokens, partials folded in a fixed order
  const int S = route_bwd_splits(desc);
  GemmArgs p = blank();
  p.a = opnd(dlogits, E, 0, 1);
  p.b = opnd(x, desc->d, 0, 1);
  p.c = S > 1 ? ws : (void*)dw_r;
  p.ldc = desc->d;
  p.G = 1;
  p.M = E;
  p.N = desc->d;
  p.K = T;
  p.k_splits = S;
  {
    Scope sc(K_ROUTER_DW, s);
    MOE_TRY(hip_check(gemm_router_dw(p, desc->dtype == MOE_BF16, s), "router dw"));
  }
  if (S > 1) {
    Scope sc(K_ROUTER_DW_REDUCE, s);
    MOE_TRY(hip_check(launch_splitk_reduce((const float*)ws, S, (int64_t)E * desc->d, dw_r, s),
                      "router dw reduce"));
  }
  }
  if ((aux_coef != 0.0f || z_coef != 0.0f) && router_x3_bwd_splits(desc) && router_x3_dense_dx(desc)) {
    // A' = [dl_hi | dl_hi | dl_mid | dl_hi | dl_mid | dl_lo] (T x 6E) against
    // B' = [W_hi; W_mid; W_hi; W_lo; W_mid; W_hi] (6E x d, read K-strided);
    // term codes per block, two bits each from block 0 up
    const int64_t d = desc->d;
    bf16_t* a6 = (bf16_t*)ws;
    bf16_t* b6 = (bf16_t*)((char*)ws + align256((size_t)T * 6 * E * 2));
    const int code_a = 0 | 0 << 2 | 1 << 4 | 0 << 6 | 1 << 8 | 2 << 10;
    const int code_b = 0 | 1 << 2 | 0 << 4 | 2 << 6 | 1 << 8 | 0 << 10;
    {
      Scope sc(K_ROUTER_SPLIT, s);
      MOE_TRY(hip_check(launch_split_bf16x3(dlogits, T, E, a6, 6 * E, E, s, 6, code_a),
                        "router dlogits split (dx)"));
      MOE_TRY(hip_check(launch_split_bf16x3(w_r, E, d, b6, d, E * d, s, 6, code_b),
                        "router weight split (dx)"));
    }
    GemmArgs q = blank();
    q.a = opnd(a6, 6 * E, 0, 0);
    q.b = opnd(b6, d, 0, 0);
    q.c = dx_router;
    q.ldc = d;
    q.G = 1;
    q.M = T;
    q.N = d;
    q.K = 6 * E;
    Scope sc(K_ROUTER_DX, s);
    return hip_check(gemm_bf16(q, true, false, EPI_STORE_F32, RAG_NONE, s), "router dx");
  }
  Scope sc(K_ROUTER_DX, s);
  // dx_router = dl W_r; dl is nonzero only on the chosen experts unless a loss term is dense
  if (aux_coef == 0.0f && z_coef == 0.0f)
    return hip_check(launch_router_dx_sparse(dlogits, topk_idx, w_r, T, E, k, desc->d, dx_router, s),
                     "router dx");
  GemmArgs q = blank();
  q.a = opnd(dlogits, E, 0, 1);
  q.b = opnd(w_r, desc->d, 0, 0);
  q.c = dx_router;
  q.ldc = desc->d;
  q.G = 1;
  q.M = T;
  q.N = desc->d;
  q.K = E;
  return hip_check(gemm_router_dx(q, s), "router dx");
}

int moe_permute_bwd(const moe_desc* desc, const void* dx_perm, const int32_t* row_of,
                    const void* dx_shared, const float* dx_router, void* dx, void* stream) {
  g_err[0] = 0;
  MOE_TRY(check_desc(desc));
  MOE_TRY(need(dx_perm, "dx_perm"));
  MOE_TRY(need(row_of, "row_of"));
  MOE_TRY(opt(dx_shared, "dx_shared"));
  MOE_TRY(opt(dx_router, "dx_router"));
  MOE_TRY(need(dx, "dx"));
  if (desc->T == 0) return MOE_OK;
  Scope sc(K_UNPERMUTE, (hipStream_t)stream);
  return hip_check(launch_unpermute(dx_perm, row_of, dx_shared, dx_router,
                                    desc->dtype == MOE_BF16, (int)desc->T, (int)desc->k, desc->d,
                                    dx, (hipStream_t)stream),
                   "un-permute");
}

}  // extern "C"
