/*
 * moe.h - C ABI of libmoe: one Mixture-of-Experts layer, forward and backward,
 * on one AMD Instinct MI355X (gfx950).
 *
 * Pages cited (titles as printed on them):
 *   [Recipe]  "MoE 训练加速实战：DeepEP + Grouped GeMM + Aux-Loss-Free 的 Qwen3.5 配方"
 *   [Balance] "负载均衡策略：MoE训练稳定性保障"
 *   [ETP]     "ETP专家并行加速MoE模型：ms-swift中稀疏架构的极致优化"
 *   [VPP]     "MoE模型训练加速10倍？看ms-swift如何通过ETP和VPP实现突破"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers. `desc` and the size/out-parameters of the utility calls are host
 *   pointers. Every tensor pointer is a device pointer (HBM), 16-byte aligned,
 *   row-major and densely packed with the shape given below. The caller
 *   allocates and frees every buffer; the library never allocates, frees or
 *   keeps a pointer after a call returns. Scratch memory comes from the
 *   caller's workspace `ws` of at least moe_workspace_size(desc, op) bytes
 *   (moe_permute_noalloc alone uses a library-owned device array instead).
 * Dtypes. "dt" means the layer dtype desc->dtype (MOE_F32: float, MOE_BF16:
 *   bfloat16 bit patterns). Router weight, biases, scores, gates, dgate,
 *   statistics, logits and their gradients are always float32. Indices,
 *   counts and offsets are int32.
 * Weights are stored out x in (the product is x W^T): router W_r [E, d];
 *   expert first matrix w13 [E, 2f, d] for SwiGLU (rows [0,f) gate W1, rows
 *   [f,2f) up W3) or w1 [E, f, d] for GELU; down matrix w2 [E, d, f]. The
 *   shared expert (desc->n_shared == 1) has sw13 [1, 2f, d] / [1, f, d] and
 *   sw2 [1, d, f].
 * Routed rows. Kept assignments are laid out expert-major and, inside an
 *   expert, by ascending token ("rows"). Buffers of routed rows are sized for
 *   the worst case T*k rows; only the first A = offsets[E] rows are written
 *   or read, so no device-to-host read is ever needed.
 * Streams. Every call enqueues its kernels on `stream` (a hipStream_t, NULL =
 *   the null stream) and returns without synchronising. Outputs are written,
 *   never accumulated into. Results are deterministic: the same inputs give
 *   the same bits (no floating-point atomics; fixed summation orders).
 * Errors. Every call returns a moe_status. Arguments are validated before any
 *   HIP call; on failure nothing is enqueued and moe_last_error() (a
 *   thread-local string) says why. A launch failure returns MOE_ERR_HIP.
 *   Device faults surface at the caller's next synchronisation. T == 0 is a
 *   successful no-op. No C++ exception crosses this ABI.
 * Limits. 1 <= k <= E <= 1024; n_shared in {0, 1}; d and f multiples of 8;
 *   T*k < 2^31.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 7

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad shape or enum */
  MOE_ERR_UNSUPPORTED = 2,   /* valid but not implemented combination */
  MOE_ERR_WORKSPACE = 3,     /* ws smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
typedef enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 } moe_score_fn;
typedef enum { MOE_SWIGLU = 0, MOE_GELU = 1 } moe_activation;
typedef enum { MOE_FP8_E4M3 = 0, MOE_FP8_E5M2 = 1 } moe_fp8_format;

/* Layer description (host struct, read during the call only). */
typedef struct {
  int64_t T;         /* tokens */
  int64_t d;         /* model width */
  int64_t E;         /* routed experts */
  int64_t k;         /* experts per token */
  int64_t f;         /* expert hidden width (d_ff) */
  int64_t n_shared;  /* always-on shared experts: 0 or 1 */
  int32_t dtype;     /* moe_dtype */
  int32_t score;     /* moe_score_fn */
  int32_t act;       /* moe_activation */
  float gumbel_tau;  /* noisy-gate temperature ([Balance], section 噪声注入);
                        0 = plain router, > 0 = moe_route takes Gumbel uniforms */
  int64_t capacity;  /* per-expert limit on kept assignments; < 0: no limit */
  int32_t fp8_grad;  /* moe_fp8_format of the FP8 backward's gradient operands
                        (dO, dpre): E4M3 (0, the default) or E5M2 (1); the
                        weights and activations are E4M3 either way */
  int32_t reserved;  /* 0 */
} moe_desc;

/* Which call a workspace is for (moe_workspace_size). */
typedef enum {
  MOE_OP_ROUTE = 0,
  MOE_OP_AUX_STATS = 1,
  MOE_OP_PERMUTE = 2,
  MOE_OP_FFN_FWD = 3,
  MOE_OP_FFN_BWD = 4,
  MOE_OP_ROUTE_BWD = 5,
  MOE_OP_FFN_FWD_FP8 = 6,
  MOE_OP_FFN_BWD_FP8 = 7,
  MOE_OP_FFN_FWD_FP8B = 8,
  MOE_OP_FFN_BWD_FP8W = 9,
  MOE_OP_FFN_BWD_FP8B = 10,
  MOE_OP_FFN_BWD_FP8BW = 11
} moe_op;

/* ---------------------------------------------------------------- router
 * moe_route: [Recipe] §2.2 (router math): logits l = x W_r^T (+ logit_bias),
 * computed in float32 ([Recipe] §1 and §9.2: router kept in fp32);
 * in a bf16 layer with E > 8 and E a multiple of 8 the product runs on the
 * bf16 matrix cores over an exact three-term bf16 split of W_r (each
 * product x * term is exact, sums are float32), otherwise on float32 ones;
 * scores s = softmax(l) (max-subtracted) or sigmoid(l); selection key
 * s (+ sel_bias, the aux-loss-free bias of [Recipe] §5.3 that steers top-k
 * only); the k experts with the largest keys, ties to the lower index, kept
 * in rank order; gate weights renormalised over the chosen k from the
 * unbiased scores: g_j = s_{e_j} / sum_j' s_{e_j'}.
 *   x          [T, d] dt                     in
 *   w_r        [E, d] float                  in
 *   logit_bias [E] float or NULL             in  (added to the logits)
 *   sel_bias   [E] float or NULL             in  (added to the key only)
 *   gumbel_u   [T, E] float in [0, 1)        in  (required iff desc->gumbel_tau > 0)
 * Noisy gate ([Balance], section 噪声注入): with desc->gumbel_tau = tau > 0
 * the logits become (l + g) / tau, g = -log(-log(u + 1e-10) + 1e-10) (g is
 * evaluated in float64 from the float32 draw); scores, key, gates and lse all
 * use them. Softmax scoring only (sigmoid returns MOE_ERR_UNSUPPORTED). The
 * caller draws u, so the noise is reproducible and testable.
 *   topk_idx   [T, k] int32                  out (expert of each slot)
 *   gate       [T, k] float                  out
 *   scores     [T, E] float                  out
 *   lse        [T] float or NULL             out (log sum_e exp(l_te), for the z-loss)
 *   ws         MOE_OP_ROUTE bytes            scratch (E > 8: the logits, and the
 *              partial products of x W_r^T: split-K partials, or for the
 *              bf16 split the three terms of W_r and their products)
 */
int moe_route(const moe_desc* desc, const void* x, const float* w_r, const float* logit_bias,
              const float* sel_bias, const float* gumbel_u, int32_t* topk_idx, float* gate,
              float* scores, float* lse, void* ws, size_t ws_bytes, void* stream);

/* moe_aux_stats: load-balance statistics of [Balance] (section 辅助损失函数)
 * and [Recipe] §5.2: counts_i = assignments routed to expert i before any
 * capacity drop; y_i = counts_i / (T k); z_i = mean over tokens of s_ti;
 * out3[0] = S = sum_i y_i z_i; out3[1] = L_aux = E * S; out3[2] = router
 * z-loss mean_t lse_t^2 when lse is given, else 0 (the z-loss is named with
 * weight 1e-3 in [Recipe] §9.1 but not defined there; this is the common
 * definition). Sums run in a fixed order (deterministic).
 *   scores [T, E] float, topk_idx [T, k] int32, lse [T] float or NULL   in
 *   counts [E] int32, y [E] float, z [E] float, out3 [3] float           out
 */
int moe_aux_stats(const moe_desc* desc, const float* scores, const int32_t* topk_idx,
                  const float* lse, int32_t* counts, float* y, float* z, float* out3, void* ws,
                  size_t ws_bytes, void* stream);

/* moe_bias_update: the aux-loss-free balancing step of [Recipe] §5.4:
 * b_i <- b_i + gamma * sign(1/E - f_i) with the load f_i = counts_i / (T k);
 * an exactly balanced expert keeps b_i. The comparison is exact
 * (counts_i * E against T * k). In place on `bias`.
 *   counts [E] int32 (from moe_aux_stats)   in
 *   bias   [E] float                         in/out (the sel_bias of moe_route)
 */
int moe_bias_update(const moe_desc* desc, const int32_t* counts, float gamma, float* bias,
                    void* stream);

/* ---------------------------------------------------------------- permute
 * moe_permute: local dispatch ([Recipe] §3.2; [Balance] section 负载感知调度,
 * tokens sorted by destination expert before the exchange) with the capacity
 * limit of [Balance] section 专家容量裁剪: assignment (t, j) to expert e is
 * kept when fewer than desc->capacity earlier tokens were routed to e.
 * Histogram -> exclusive scan -> stable scatter; the row order is fixed by
 * (expert, token), never by thread timing.
 *   x         [T, d] dt                     in
 *   topk_idx  [T, k] int32                  in
 *   offsets   [E + 1] int32                 out (rows of expert e: [offsets[e], offsets[e+1]))
 *   row_of    [T, k] int32                  out (row of (t, j), or -1 if dropped)
 *   token_of  [T*k] int32                   out (token of each row; first A entries)
 *   n_dropped [1] int32                     out (T*k - A)
 *   x_perm    [T*k, d] dt                   out (x_perm[row] = x[token_of[row]]; first A rows)
 */
int moe_permute(const moe_desc* desc, const void* x, const int32_t* topk_idx, int32_t* offsets,
                int32_t* row_of, int32_t* token_of, int32_t* n_dropped, void* x_perm, void* ws,
                size_t ws_bytes, void* stream);

/* moe_permute_noalloc: moe_permute with no workspace argument, for callers
 * that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, results and errors as
 * moe_permute (bit-identical outputs); the permute's scratch (its per-block
 * base counts, at most 128 KiB) lives in a library-owned device array, one
 * per GPU, held until the process ends. It allocates nothing: the array's
 * address is looked up once per device on the first call there.
 * Every call on one GPU uses that GPU's one array, so calls that overlap on
 * one GPU (other streams or threads) race and must be serialised by the
 * caller. A size that would need more scratch returns MOE_ERR_UNSUPPORTED
 * (the permute chooses its token blocks so that it never does). */
int moe_permute_noalloc(const moe_desc* desc, const void* x, const int32_t* topk_idx,
                        int32_t* offsets, int32_t* row_of, int32_t* token_of, int32_t* n_dropped,
                        void* x_perm, void* stream);

/* ------------------------------------------------------------ grouped FFN
 * moe_grouped_ffn_fwd: the grouped GEMM of [Recipe] §4.2 - every expert's FFN
 * on its own contiguous rows in one launch per matrix - for the two-matrix
 * expert of [ETP] (up-projection then down-projection): SwiGLU
 * H = silu(X W1^T) * (X W3^T) or GELU H = gelu(X W1^T) (exact erf form),
 * O = H W2^T. bf16 in, float32 accumulate, dt out. The shared expert
 * ([Recipe] §2.3 / §9.1) runs on all T rows of x when desc->n_shared == 1.
 *   x_perm   [T*k, d] dt, offsets [E+1] int32 (from moe_permute)   in
 *   x        [T, d] dt (shared expert input; NULL if n_shared == 0) in
 *   w13, w2  routed weights; sw13, sw2 shared weights or NULL       in
 *   save_pre [T*k, 2f] (SwiGLU: [a | b]) or [T*k, f] (GELU: a) dt   out (for the backward)
 *   save_h   [T*k, f] dt                                            out (H, for the backward)
 *   save_pre_s, save_h_s: the same for the shared expert ([T, ...]) out or NULL
 *   out      [T*k, d] dt                                            out (O per row)
 *   out_shared [T, d] dt or NULL                                    out
 *   ws       MOE_OP_FFN_FWD bytes: bf16 splits the down-projection's last,
 *            partial round of tiles over K, and keeps its partial sums and
 *            counters here (fp32: none)                             scratch
 */
int moe_grouped_ffn_fwd(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                        const void* x, const void* w13, const void* w2, const void* sw13,
                        const void* sw2, void* save_pre, void* save_h, void* save_pre_s,
                        void* save_h_s, void* out, void* out_shared, void* ws, size_t ws_bytes,
                        void* stream);

/* ------------------------------------------------------------ FP8 forward
 * [Recipe] §8.1 and §9.1 run the forward GEMMs in FP8 with bf16 activations;
 * §6.2 keeps experts in FP8 storage and widens them for use. Format and
 * granularity are not given there; this library uses OCP E4M3 codes with one
 * power-of-two scale per row of each K-contiguous operand.
 *
 * moe_quantize_fp8: row i of a bf16 matrix ->
 *   codes[i][k] = E4M3 nearest (ties to even) of src[i][k] * 2^-scale_exp[i],
 *   scale_exp[i] = smallest integer e with max_k |src[i][k]| <= 448 * 2^e
 *   (0 for an all-zero row), so src[i][k] ~= e4m3(codes[i][k]) * 2^scale_exp[i].
 * The scaling is exact; the codes are a bit-exact function of the input.
 * Inputs must be finite. No desc: a plain matrix operation.
 *   src        [rows, K] bf16, row stride ld_src elements (multiple of 8)   in
 *   valid_rows device int32 or NULL: rows >= *valid_rows are left untouched
 *              (e.g. offsets + E, the routed row count)                     in
 *   codes      [rows, K] uint8, row stride ld_codes bytes (multiple of 16)  out
 *   scale_exp  [rows] int32                                                 out
 * K must be a positive multiple of 16; rows < 2^31.
 */
int moe_quantize_fp8(const void* src, int64_t rows, int64_t K, int64_t ld_src,
                     const int32_t* valid_rows, void* codes, int64_t ld_codes, int32_t* scale_exp,
                     void* stream);

/* moe_grouped_ffn_fwd_fp8: moe_grouped_ffn_fwd with both GEMMs on FP8
 * operands (moe_quantize_fp8 codes and exponents). The up-projection takes
 * the quantized rows of x_perm and of w13 (one exponent per weight row), the
 * pre-activations and H are written in bf16 as in moe_grouped_ffn_fwd (the
 * backward runs on them, in bf16, against the bf16 weights); the bf16 H is
 * then quantized per row into the workspace and the down-projection takes it
 * with the quantized rows of w2. Each output element is
 * 2^(e_row + e_weight_row) * sum_k e4m3 * e4m3, accumulated in float32.
 * desc->dtype must be MOE_BF16; d and f multiples of 16.
 *   xq_perm [T*k, d] uint8, sx_perm [T*k] int32 (rows below offsets[E])   in
 *   xq [T, d] uint8, sx [T] int32: quantized x for the shared expert       in (or NULL)
 *   w13q [E, P, d] uint8, s13 [E, P] int32 (P = 2f SwiGLU, f GELU)         in
 *   w2q [E, d, f] uint8, s2 [E, d] int32                                   in
 *   sw13q, ss13, sw2q, ss2: the shared expert's, or NULL                   in
 *   save_pre, save_h, save_pre_s, save_h_s, out, out_shared: as in
 *     moe_grouped_ffn_fwd (bf16)                                           out
 *   ws         MOE_OP_FFN_FWD_FP8 bytes (H codes and exponents, then the
 *              down-projection's split-K partials for its last round)  scratch
 */
int moe_grouped_ffn_fwd_fp8(const moe_desc* desc, const void* xq_perm, const int32_t* sx_perm,
                            const int32_t* offsets, const void* xq, const int32_t* sx,
                            const void* w13q, const int32_t* s13, const void* w2q,
                            const int32_t* s2, const void* sw13q, const int32_t* ss13,
                            const void* sw2q, const int32_t* ss2, void* save_pre, void* save_h,
                            void* save_pre_s, void* save_h_s, void* out, void* out_shared, void* ws,
                            size_t ws_bytes, void* stream);

/* Block scales. [Recipe] §8.1 and §9.1 leave the FP8 scaling granularity
 * open; the second FP8 mode reads it as one power-of-two scale per block of
 * 32 consecutive elements along K of each operand row (the finest granularity
 * the gfx950 block-scaled matrix instructions take), with the per-row rule of
 * moe_quantize_fp8 applied to each block and the exponent clipped to
 * [-127, 127].
 *
 * moe_quantize_fp8_blocks: row i, block b = k / 32 of a bf16 matrix ->
 *   e[i][b] = clip(smallest integer e with max over the block |src| <= 448 * 2^e,
 *                  -127, 127) (0 for an all-zero block),
 *   codes[i][k] = E4M3 nearest (ties to even) of src[i][k] * 2^-e[i][k/32],
 *   and the byte e[i][b] + 127 (the e8m0 encoding) in the scales.
 * Scale layout: the bytes of blocks 4w .. 4w+3 of row i form 32-bit word w
 * (low byte first; w < KW = ceil(K / 128); bytes of blocks at or past K
 * hold 127, a scale of 1), and the words are 32-row interleaved: word w of
 * row i is word (i / 32 * KW + w) * 32 + i % 32 of the array, so one 128-k
 * step of 32 consecutive rows is one 128-byte line. The array holds
 * MOE_FP8_BLOCK_SCALE_BYTES(rows, K) = 128 * KW * ceil(rows / 32) bytes; the
 * words of the padding rows of the last group of 32 are left untouched.
 * A last block shorter than 32 (K % 32 == 16) takes its max over what is
 * there. The codes and bytes are a bit-exact function of the input; inputs
 * must be finite. No desc: a plain matrix operation.
 *   src        [rows, K] bf16, row stride ld_src elements (multiple of 8)   in
 *   valid_rows device int32 or NULL: rows >= *valid_rows are left untouched in
 *   codes      [rows, K] uint8, row stride ld_codes bytes (multiple of 16)  out
 *   scales     MOE_FP8_BLOCK_SCALE_BYTES(rows, K) bytes, layout above       out
 * K must be a positive multiple of 16; rows < 2^31; the scale array must
 * stay under 2^31 words.
 */
#define MOE_FP8_BLOCK_SCALE_BYTES(rows, K) \
  ((size_t)128 * (size_t)(((K) + 127) / 128) * (size_t)(((rows) + 31) / 32))
int moe_quantize_fp8_blocks(const void* src, int64_t rows, int64_t K, int64_t ld_src,
                            const int32_t* valid_rows, void* codes, int64_t ld_codes,
                            uint8_t* scales, void* stream);

/* moe_grouped_ffn_fwd_fp8b: moe_grouped_ffn_fwd_fp8 with block scales
 * (moe_quantize_fp8_blocks codes and scale arrays) in place of per-row
 * exponents. Each output element is the sum over blocks b of
 * 2^(e_row[b] + e_weight_row[b]) * sum_{k in b} e4m3 * e4m3, accumulated in
 * float32 (the block-scaled MFMA applies both scales to each 32-k product).
 * H is quantized with block scales into the workspace between the GEMMs.
 * Weight scale arrays are those of the [E * rows, K] matrix (expert e's row
 * n is matrix row e * rows + n). desc->dtype must be MOE_BF16; d and f
 * multiples of 16. SB(r, K) = MOE_FP8_BLOCK_SCALE_BYTES(r, K).
 *   xq_perm [T*k, d] uint8, bx_perm SB(T*k, d) bytes                      in
 *   xq [T, d] uint8, bx SB(T, d) bytes: the shared expert's x             in (or NULL)
 *   w13q [E, P, d] uint8, b13 SB(E*P, d) bytes                            in
 *   w2q [E, d, f] uint8, b2 SB(E*d, f) bytes                              in
 *   sw13q, sb13 (SB(P, d)), sw2q, sb2 (SB(d, f)): the shared expert's,
 *     or NULL                                                             in
 *   save_pre, save_h, save_pre_s, save_h_s, out, out_shared: as in
 *     moe_grouped_ffn_fwd (bf16)                                          out
 *   ws         MOE_OP_FFN_FWD_FP8B bytes (H codes and block scales, then
 *              the down-projection's split-K partials)                 scratch
 */
int moe_grouped_ffn_fwd_fp8b(const moe_desc* desc, const void* xq_perm, const uint8_t* bx_perm,
                             const int32_t* offsets, const void* xq, const uint8_t* bx,
                             const void* w13q, const uint8_t* b13, const void* w2q,
                             const uint8_t* b2, const void* sw13q, const uint8_t* sb13,
                             const void* sw2q, const uint8_t* sb2, void* save_pre, void* save_h,
                             void* save_pre_s, void* save_h_s, void* out, void* out_shared,
                             void* ws, size_t ws_bytes, void* stream);

/* moe_grouped_ffn_bwd: backward of moe_grouped_ffn_fwd ([VPP]: each device
 * runs forward and backward of its local experts between the exchanges).
 * dgrad: dH = dO W2; SwiGLU da = dH * b * silu'(a), db = dH * silu(a)
 * (GELU da = dH * gelu'(a)); dX = [da db] W13. wgrad: dW2 = dO^T H,
 * dW13 = [da db]^T X. The shared expert's upstream gradient is dy itself.
 * Gradients are written in dt (an expert with no rows gets dW = 0).
 *   dout [T*k, d] dt (from moe_combine_bwd), dy [T, d] dt (shared; may be NULL if n_shared == 0)
 *   dx_perm [T*k, d] dt, dx_shared [T, d] dt or NULL                out
 *   dw13, dw2 (routed weight shapes), dsw13, dsw2 or NULL           out
 *   ws   MOE_OP_FFN_BWD bytes: dpre, then (bf16) the dX GEMM's split-K
 *        partials for its last round of tiles                        scratch
 */
int moe_grouped_ffn_bwd(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                        const void* x, const void* w13, const void* w2, const void* sw13,
                        const void* sw2, const void* save_pre, const void* save_h,
                        const void* save_pre_s, const void* save_h_s, const void* dout,
                        const void* dy, void* dx_perm, void* dx_shared, void* dw13, void* dw2,
                        void* dsw13, void* dsw2, void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------- FP8 backward
 * [Megatron10x] §5.2 trains in FP8 mixed precision, and [Recipe] §8.1 and
 * §9.1 list FP8 training with bf16 activations. The pages do not say which
 * backward GEMMs run in FP8. Reading taken here: the two data-gradient GEMMs
 * use the forward's per-row scheme, and the weight gradients, which reduce
 * over tokens, stay in bf16. A data gradient reads a weight along its input
 * dimension, so the weight enters transposed and is quantized per input
 * channel.
 *
 * moe_quantize_fp8_t: moe_quantize_fp8 applied to the rows of the transposes
 * of G row-major R x C bf16 matrices. Codes and exponents are a bit-exact
 * function of the input:
 *   codes[g][c][r] = E4M3 nearest (ties to even) of src[g][r][c] * 2^-scale_exp[g][c]
 *   scale_exp[g][c] = smallest e with max_r |src[g][r][c]| <= 448 * 2^e
 *                     (0 for an all-zero column)
 * Inputs must be finite. No desc: a plain matrix operation.
 *   src        [G, R, C] bf16     in
 *   codes      [G, C, R] uint8    out
 *   scale_exp  [G, C] int32       out
 * Constraints: R a multiple of 16 in [16, 2^22]; C a multiple of 8 in [8, 2^31);
 * 0 <= G <= 65535; every pointer 16-byte aligned.
 */
int moe_quantize_fp8_t(const void* src, int64_t G, int64_t R, int64_t C, void* codes,
                       int32_t* scale_exp, void* stream);

/* moe_quantize_fp8_both: moe_quantize_fp8 of the rows of G row-major R x C
 * bf16 matrices and moe_quantize_fp8_t of their columns, with the same codes
 * and exponents as the two separate calls. It takes two reads of src instead
 * of three: the row pass also keeps per-column maxima (a partial per 64 rows,
 * in ws), then the transposes are written with the column exponents. It is
 * for a layer whose forward and data gradients both run in FP8: the forward
 * quantizes each weight this way, and the backward uses the transposed codes.
 *   src          [G, R, C] bf16                          in
 *   codes        [G, R, C] uint8, scale_exp [G, R] int32  out (rows)
 *   codes_t      [G, C, R] uint8, scale_exp_t [G, C] int32 out (columns)
 *   ws           G * ceil(R / 64) * C * 2 bytes, rounded up to a multiple of
 *                256, 256-byte aligned                    scratch
 * Constraints: R a multiple of 16 in [16, 2^22]; C a multiple of 16 in
 * [16, 32768]; 0 <= G <= 65535; src, codes and exponent pointers 16-byte aligned.
 */
int moe_quantize_fp8_both(const void* src, int64_t G, int64_t R, int64_t C, void* codes,
                          int32_t* scale_exp, void* codes_t, int32_t* scale_exp_t, void* ws,
                          size_t ws_bytes, void* stream);

/* Square-block weights. The pages fix no scale granularity for the weights
 * either; the third FP8 mode quantizes each weight matrix once in 32 x 32
 * squares (rows x columns of the stored matrix, from its first row and
 * column, the last ones partial), each with the block rule of
 * moe_quantize_fp8_blocks on the square's maximum. A square is a 1 x 32
 * block of every row it covers in the matrix and in its transpose, so the
 * forward (rows) and the data gradients (the transpose) share one
 * quantization.
 *
 * moe_quantize_fp8_squares: for G row-major R x C bf16 matrices,
 *   e[g][i][j] = clip(smallest integer e with max over square (i, j) of
 *                     |src[g]| <= 448 * 2^e, -127, 127) (0 for an all-zero square),
 *   codes[g][r][c] = codes_t[g][c][r] = E4M3 nearest (ties to even) of
 *                    src[g][r][c] * 2^-e[g][r/32][c/32],
 * and the block-scale bytes of both layouts: scales as moe_quantize_fp8_blocks
 * writes them for the [G*R, C] matrix of codes (row g*R + r, block c/32 holds
 * e[g][r/32][c/32] + 127), scales_t for the [G*C, R] matrix of codes_t (row
 * g*C + c, block r/32). One read of src writes both. Bit-exact function of
 * the input; inputs must be finite. No desc: a plain matrix operation.
 *   src       [G, R, C] bf16                                          in
 *   codes     [G, R, C] uint8, scales MOE_FP8_BLOCK_SCALE_BYTES(G*R, C) out
 *   codes_t   [G, C, R] uint8, scales_t MOE_FP8_BLOCK_SCALE_BYTES(G*C, R) out
 * Either layout may be skipped: codes and scales both NULL (only the
 * transposes, for FP8 data gradients after a bf16 forward), or codes_t and
 * scales_t both NULL (only the rows, for an FP8 forward alone); not both.
 * Constraints: R and C multiples of 16 in [16, 2^22]; 0 <= G <= 65535; each
 * scale array under 2^31 words; every pointer 16-byte aligned.
 */
int moe_quantize_fp8_squares(const void* src, int64_t G, int64_t R, int64_t C, void* codes,
                             uint8_t* scales, void* codes_t, uint8_t* scales_t, void* stream);

/* moe_grouped_ffn_bwd_fp8: moe_grouped_ffn_bwd with its two data-gradient
 * GEMMs on FP8 operands. Per group:
 *   1. the upstream gradient rows are quantized per row;
 *   2. dH = dO W2 runs against w2q_t, and the activation backward in its
 *      epilogue writes the pre-activation gradient (dpre) in bf16;
 *   3. that bf16 dpre is quantized per row;
 *   4. dX = dpre W13 runs against w13q_t.
 * Each GEMM output element is 2^(e_row + e_channel) * sum_k e4m3 * e4m3,
 * accumulated in float32. The weight gradients dW2 = dO^T H and
 * dW13 = dpre^T X run in bf16 on the bf16 values, as in moe_grouped_ffn_bwd.
 * With desc->fp8_grad = MOE_FP8_E5M2 the two gradient operands (dO, dpre)
 * are quantized to OCP E5M2 instead (the same per-row rule with 57344 =
 * 1.75 * 2^15 in place of 448; the hybrid scheme of FP8 training recipes,
 * a reading: the pages name no format), against the E4M3 weights.
 * desc->dtype must be MOE_BF16; d and f must be multiples of 16.
 *   w2q_t [E, f, d] uint8, s2_t [E, f] int32    (moe_quantize_fp8_t of w2 [E, d, f])    in
 *   w13q_t [E, d, P] uint8, s13_t [E, d] int32  (moe_quantize_fp8_t of w13 [E, P, d])   in
 *   sw2q_t, ss2_t, sw13q_t, ss13_t: the shared expert's, or NULL                       in
 *   the other arguments are as in moe_grouped_ffn_bwd
 *   ws  MOE_OP_FFN_BWD_FP8 bytes (moe_grouped_ffn_bwd's layout: dpre and the dX GEMM's
 *       split-K partials; then the FP8 codes and exponents)                            scratch
 */
int moe_grouped_ffn_bwd_fp8(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                            const void* x, const void* w13q_t, const int32_t* s13_t,
                            const void* w2q_t, const int32_t* s2_t, const void* sw13q_t,
                            const int32_t* ss13_t, const void* sw2q_t, const int32_t* ss2_t,
                            const void* save_pre, const void* save_h, const void* save_pre_s,
                            const void* save_h_s, const void* dout, const void* dy, void* dx_perm,
                            void* dx_shared, void* dw13, void* dw2, void* dsw13, void* dsw2,
                            void* ws, size_t ws_bytes, void* stream);

/* moe_grouped_ffn_bwd_fp8w: moe_grouped_ffn_bwd_fp8 with the weight
 * gradients on FP8 operands as well. [Megatron10x] §5.2 trains in FP8 mixed
 * precision without naming the GEMMs; the reading taken here quantizes the
 * operands of dW2 = dO^T H and dW13 = dpre^T X (the stored bf16 values) per
 * column, with one power-of-two scale per block of 32 consecutive tokens of
 * each expert (blocks start at the expert's first row, the last may be
 * partial; the rule of moe_quantize_fp8_blocks along the token axis). The
 * library writes each operand's transpose in FP8 into the workspace, each
 * expert's tokens starting on a 128-token step, and runs the block-scaled
 * GEMM over them: each output element is the sum over token blocks of
 * 2^(e_a + e_b) * sum e4m3 * e4m3, accumulated in float32, stored in bf16.
 * desc->fp8_grad selects the gradient operands' format (dO, dpre) as in
 * moe_grouped_ffn_bwd_fp8; H and X stay E4M3.
 * Arguments as in moe_grouped_ffn_bwd_fp8.
 *   ws  MOE_OP_FFN_BWD_FP8W bytes (moe_grouped_ffn_bwd_fp8's layout, then
 *       the token-axis codes and scales of the weight gradients' operands:
 *       about (max(d, 2f|f) + max(f, d)) * (T*k + 128 E) bytes)            scratch
 */
int moe_grouped_ffn_bwd_fp8w(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                             const void* x, const void* w13q_t, const int32_t* s13_t,
                             const void* w2q_t, const int32_t* s2_t, const void* sw13q_t,
                             const int32_t* ss13_t, const void* sw2q_t, const int32_t* ss2_t,
                             const void* save_pre, const void* save_h, const void* save_pre_s,
                             const void* save_h_s, const void* dout, const void* dy, void* dx_perm,
                             void* dx_shared, void* dw13, void* dw2, void* dsw13, void* dsw2,
                             void* ws, size_t ws_bytes, void* stream);

/* moe_grouped_ffn_bwd_fp8b: moe_grouped_ffn_bwd_fp8 with block scales (the
 * square mode's data gradients). The upstream gradient rows and the bf16 dpre
 * are quantized with moe_quantize_fp8_blocks' rule along their reduction axis
 * (d for dH, P for dX; E4M3 or, with desc->fp8_grad = MOE_FP8_E5M2, E5M2),
 * and the weight operands are the transposed square-block codes of
 * moe_quantize_fp8_squares. Each output element of dH and dX is the sum over
 * blocks b of 2^(e_grad[b] + e_weight[b]) * sum_{k in b} code * code,
 * accumulated in float32. The weight gradients run in bf16 as in
 * moe_grouped_ffn_bwd_fp8. SB(r, K) = MOE_FP8_BLOCK_SCALE_BYTES(r, K).
 *   w2q_t [E, f, d] uint8, b2_t SB(E*f, d) bytes  (codes_t, scales_t of
 *     moe_quantize_fp8_squares on w2 [E, d, f])                              in
 *   w13q_t [E, d, P] uint8, b13_t SB(E*d, P) bytes (the same on w13 [E, P, d]) in
 *   sw2q_t, sb2_t (SB(f, d)), sw13q_t, sb13_t (SB(d, P)): the shared
 *     expert's, or NULL                                                      in
 *   the other arguments are as in moe_grouped_ffn_bwd_fp8
 *   ws  MOE_OP_FFN_BWD_FP8B bytes (moe_grouped_ffn_bwd's layout, then the
 *       FP8 codes and block scales of dO and dpre)                     scratch
 */
int moe_grouped_ffn_bwd_fp8b(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                             const void* x, const void* w13q_t, const uint8_t* b13_t,
                             const void* w2q_t, const uint8_t* b2_t, const void* sw13q_t,
                             const uint8_t* sb13_t, const void* sw2q_t, const uint8_t* sb2_t,
                             const void* save_pre, const void* save_h, const void* save_pre_s,
                             const void* save_h_s, const void* dout, const void* dy, void* dx_perm,
                             void* dx_shared, void* dw13, void* dw2, void* dsw13, void* dsw2,
                             void* ws, size_t ws_bytes, void* stream);

/* moe_grouped_ffn_bwd_fp8bw: moe_grouped_ffn_bwd_fp8b with the weight
 * gradients on token-axis FP8 operands as in moe_grouped_ffn_bwd_fp8w.
 * Arguments as in moe_grouped_ffn_bwd_fp8b.
 * dO and dpre are each read once for their row blocks and their token-axis
 * blocks.
 *   ws  MOE_OP_FFN_BWD_FP8BW bytes (moe_grouped_ffn_bwd_fp8b's layout, then
 *       the token-axis buffers of moe_grouped_ffn_bwd_fp8w, then dO's
 *       token-axis codes and scales, d * (T*k + 128 E) bytes and more)  scratch
 */
int moe_grouped_ffn_bwd_fp8bw(const moe_desc* desc, const void* x_perm, const int32_t* offsets,
                              const void* x, const void* w13q_t, const uint8_t* b13_t,
                              const void* w2q_t, const uint8_t* b2_t, const void* sw13q_t,
                              const uint8_t* sb13_t, const void* sw2q_t, const uint8_t* sb2_t,
                              const void* save_pre, const void* save_h, const void* save_pre_s,
                              const void* save_h_s, const void* dout, const void* dy, void* dx_perm,
                              void* dx_shared, void* dw13, void* dw2, void* dsw13, void* dsw2,
                              void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- combine
 * moe_combine: the weighted sum of [Recipe] §2.1/§2.2 (the combine step of
 * [Recipe] §3.2): y[t] = out_shared[t] + sum over kept slots j (in slot
 * order) of gate[t,j] * out[row_of[t,j]], float32 accumulate, one rounding.
 * A dropped slot adds nothing (gates are not renormalised after a drop).
 *   out [T*k, d] dt, out_shared [T, d] dt or NULL, gate [T, k], row_of [T, k]   in
 *   y [T, d] dt                                                               out
 */
int moe_combine(const moe_desc* desc, const void* out, const void* out_shared, const float* gate,
                const int32_t* row_of, void* y, void* stream);

/* moe_combine_bwd: dgate[t,j] = <dy[t], out[row_of[t,j]]> (0 if dropped),
 * dout[row_of[t,j]] = gate[t,j] * dy[t].
 *   dy [T, d] dt, out [T*k, d] dt, gate [T, k], row_of [T, k]   in
 *   dgate [T, k] float, dout [T*k, d] dt                         out
 */
int moe_combine_bwd(const moe_desc* desc, const void* dy, const void* out, const float* gate,
                    const int32_t* row_of, float* dgate, void* dout, void* stream);

/* ------------------------------------------------------- router backward
 * moe_route_bwd: gradient of the router through the renormalised gates of
 * [Recipe] §2.2 (top-k selection itself has no gradient), plus aux_coef
 * times the gradient of L_aux = E sum_i y_i z_i with y held fixed
 * ([Recipe] §5.2; the total loss is main + lambda * aux).
 *   softmax: dl_e = g_e (dg_e - sum_j g_j dg_j) on chosen e, else 0;
 *            aux: dl_te += aux_coef (E/T) s_te (y_e - sum_i y_i s_ti)
 *   sigmoid: dl_e = s_e (1 - s_e) (dg_e - sum_j g_j dg_j) / sum_chosen s;
 *            aux: dl_te += aux_coef (E/T) y_e s_te (1 - s_te)
 * Plus z_coef times the gradient of the z-loss mean_t lse_t^2:
 *   dl_te += z_coef (2/T) lse_t softmax(l_t)_e   (softmax scoring only;
 *   z_coef != 0 with sigmoid scoring returns MOE_ERR_UNSUPPORTED).
 * With the noisy gate (desc->gumbel_tau = tau > 0) the terms above are taken
 * with respect to the noisy logits (l + g) / tau, and dlogits (the gradient
 * with respect to l) is their sum divided by tau.
 * dw_r = dl^T x, dx_router = dl W_r (float32; dw_r under the same rule
 * as moe_route's logits: in a bf16 layer with E > 8 and E % 8 == 0 it runs
 * on the bf16 matrix cores over an exact three-term bf16 split of dl; in such
 * a layer a dense dl (aux_coef or z_coef nonzero) takes dx_router there too,
 * over the six largest products of the two operands' terms).
 *   x [T, d] dt, w_r [E, d], scores [T, E], topk_idx, gate, dgate [T, k]   in
 *   y [E] float (from moe_aux_stats; may be NULL when aux_coef == 0)        in
 *   lse [T] float (from moe_route; may be NULL when z_coef == 0)            in
 *   dlogits [T, E] float, dx_router [T, d] float, dw_r [E, d] float          out
 */
int moe_route_bwd(const moe_desc* desc, const void* x, const float* w_r, const float* scores,
                  const int32_t* topk_idx, const float* gate, const float* dgate, const float* y,
                  float aux_coef, const float* lse, float z_coef, float* dlogits,
                  float* dx_router, float* dw_r, void* ws, size_t ws_bytes, void* stream);

/* moe_permute_bwd: un-permute, dx[t] = dx_shared[t] + sum over kept slots j
 * (slot order) of dx_perm[row_of[t,j]] + dx_router[t], float32 accumulate,
 * one rounding to dt.
 *   dx_perm [T*k, d] dt, row_of [T, k], dx_shared [T, d] dt or NULL,
 *   dx_router [T, d] float or NULL                                     in
 *   dx [T, d] dt                                                        out
 */
int moe_permute_bwd(const moe_desc* desc, const void* dx_perm, const int32_t* row_of,
                    const void* dx_shared, const float* dx_router, void* dx, void* stream);

/* -------------------------------------------------------------- utilities */
/* Workspace bytes `op` needs for this desc (0 is a valid answer). */
int moe_workspace_size(const moe_desc* desc, int op, size_t* bytes);
/* [Balance] section 专家容量裁剪: capacity = ceil(cf * T * k / E), evaluated
 * left to right in binary64; cf < 0 gives -1 (no limit). */
int moe_capacity(int64_t T, int64_t k, int64_t E, double cf, int64_t* capacity);
const char* moe_status_str(int status);
/* Thread-local text of the last failure on this thread ("" if none). */
const char* moe_last_error(void);
int moe_abi_version(void);

/* Per-kernel timing, for measurement and observability. While enabled
 * (on != 0), every kernel launch the library makes is bracketed by two HIP
 * timing events recorded on that launch's stream; enabling or disabling
 * drops any unread records. moe_profile_read waits for the recorded events,
 * then reports, per kernel name in first-launch order, the summed duration
 * in milliseconds and the launch count, and clears the records. Up to `cap`
 * entries are written to names/total_ms/launches (host arrays); *n receives
 * the number of distinct kernels. The name strings are static. Not meant to
 * be enabled while another thread launches through the library. */
int moe_profile_enable(int on);
int moe_profile_read(int cap, int* n, const char** names, double* total_ms, int* launches);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
