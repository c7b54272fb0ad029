"""CPU oracle of one Mixture-of-Experts layer, forward and backward.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
CPU-baseline leg may import or call this module. It shares no code with the
HIP library (no kernels, headers, helpers or constants): it is the method's
plain definition, written out in float64 NumPy so that a reader can check it
against the pages by eye. No blocking, fusion or reordering beyond what each
step states.

Pages cited (titles as printed on them):
  [Recipe]  "MoE 训练加速实战：DeepEP + Grouped GeMM + Aux-Loss-Free 的 Qwen3.5 配方"
  [Balance] "负载均衡策略：MoE训练稳定性保障"
  [ETP]     "ETP专家并行加速MoE模型：ms-swift中稀疏架构的极致优化"
  [VPP]     "MoE模型训练加速10倍？看ms-swift如何通过ETP和VPP实现突破"
  [Megatron10x] "ms-swift + Megatron：MoE模型加速10倍实测"

Readings taken where the pages are silent, garbled or disagree are listed in
the repository's design notes; each function names the one it uses.

Parity pins: every public function here is pinned by tests/test_oracle_pins.py
against a dense brute force, closed forms, invariants, central finite
differences or the worked capacity example of [Balance]; none is unpinned.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
from scipy.special import erf

NEAR_TIE = 1e-5   # fp32 score gap under which two ranks count as a near-tie


# ------------------------------------------------------------------ router
GUMBEL_EPS = 1e-10   # the eps of [Balance]'s noisy gate (section 噪声注入)


def gumbel_noise(u):
    """Gumbel noise of [Balance] (section 噪声注入) from uniforms u in [0, 1):
    g = -log(-log(u + eps) + eps). The uniforms are an input (drawn by the
    caller), so both sides see the same draws."""
    u = np.asarray(u, dtype=np.float64)
    return -np.log(-np.log(u + GUMBEL_EPS) + GUMBEL_EPS)


def router_forward(x, w_r, k, score="softmax", logit_bias=None, sel_bias=None,
                   gumbel_u=None, tau=None):
    """Router of [Recipe] §2.2: g(x) = x W_r, scores = softmax(g), top-k,
    gate weights renormalised over the chosen k.

    Noisy gate of [Balance] (section 噪声注入): with uniforms gumbel_u [T, E]
    and temperature tau, the logits become (l + gumbel_noise(u)) / tau and
    everything downstream (scores, choice, gates, statistics, z-loss) uses
    them; the returned "logits" are these. Softmax scoring only.

    x [T, d], w_r [E, d] (stored out x in, so g = x w_r^T), optional
    logit_bias [E] added to the logits (a fixed shift: it moves both the
    choice and the gate values), optional sel_bias [E] added to the scores for
    the choice only ([Recipe] §5.3, the aux-loss-free bias: b takes no gradient
    and only steers top-k; the gates use the unbiased scores).
    score="sigmoid" replaces softmax by an elementwise logistic.

    Top-k orders experts by (key descending, expert index ascending) and keeps
    the first k in that rank order.
    Returns dict(logits, scores, key, topk_idx [T,k] int64, gates [T,k]).
    """
    logits = x @ w_r.T
    if logit_bias is not None:
        logits = logits + logit_bias[None, :]
    if gumbel_u is not None:
        if score != "softmax" or not tau or tau <= 0:
            raise ValueError("the noisy gate needs softmax scoring and tau > 0")
        logits = (logits + gumbel_noise(gumbel_u)) / tau
    if score == "softmax":
        # max-subtracted so exp never overflows ([Recipe] §1: fp32 router against 0/0)
        m = logits.max(axis=1, keepdims=True)
        ex = np.exp(logits - m)
        scores = ex / ex.sum(axis=1, keepdims=True)
    elif score == "sigmoid":
        scores = 1.0 / (1.0 + np.exp(-logits))
    else:
        raise ValueError(score)
    key = scores + sel_bias[None, :] if sel_bias is not None else scores
    # stable sort on -key: equal keys keep ascending expert index
    order = np.argsort(-key, axis=1, kind="stable")
    topk_idx = order[:, :k]
    chosen = np.take_along_axis(scores, topk_idx, axis=1)
    gates = chosen / chosen.sum(axis=1, keepdims=True)
    return dict(logits=logits, scores=scores, key=key, topk_idx=topk_idx, gates=gates)


def near_tie_tokens(key, k, thresh=NEAR_TIE):
    """Tokens whose top-(k+1) keys hold an adjacent pair closer than thresh:
    there the fp32 router may legitimately order experts differently."""
    E = key.shape[1]
    srt = -np.sort(-key, axis=1)[:, : min(k + 1, E)]
    if srt.shape[1] < 2:
        return np.zeros(key.shape[0], dtype=bool)
    return (np.abs(np.diff(srt, axis=1)) < thresh).any(axis=1)


# --------------------------------------------------------------- aux stats
def aux_stats(scores, topk_idx, E):
    """Load-balance statistics of [Balance] (辅助损失函数) and [Recipe] §5.2.

    counts_i = assignments routed to expert i (before any capacity drop);
    y_i = counts_i / (T k), the fraction of routed assignments (sums to 1);
    z_i = mean over tokens of expert i's score (full pre-top-k scores);
    S = sum_i y_i z_i;  L_aux = E * S (the [Recipe] §5.2 normalisation,
    equal to 1 at uniform load). [Balance]'s own constant (N/E) * S with
    N = tokens is S times T/E, formed by the caller from S.
    """
    T, k = topk_idx.shape
    counts = np.bincount(topk_idx.ravel(), minlength=E).astype(np.int64)
    y = counts / float(T * k)
    z = scores.mean(axis=0)
    S = float((y * z).sum())
    return dict(counts=counts, y=y, z=z, S=S, L_aux=E * S)


# ---------------------------------------------------------------- capacity
def capacity(T, k, E, cf):
    """Per-expert token limit of [Balance] (专家容量裁剪): capacity_factor
    times the ideal load T k / E, rounded up. cf None -> no limit.
    The product is evaluated left to right in binary64: ((cf*T)*k)/E."""
    if cf is None:
        return None
    return int(math.ceil(cf * T * k / E))


# ----------------------------------------------------------------- permute
def permute(topk_idx, E, cap=None):
    """Local dispatch: sort assignments into expert-contiguous rows
    ([Balance] 负载感知调度: tokens pre-sorted by destination before the
    exchange; [Recipe] §3.2 dispatch). Within an expert, rows follow token
    order. With a capacity, an assignment is kept when fewer than `cap`
    earlier tokens were already routed to the same expert; the rest are
    dropped ([Balance] 专家容量裁剪).

    Returns dict(offsets [E+1], row_of [T,k] (-1 = dropped), token_of [A],
    n_dropped). x_perm = x[token_of].
    """
    T, k = topk_idx.shape
    seen = [0] * E
    kept = [[] for _ in range(E)]
    for t in range(T):
        for j in range(k):
            e = int(topk_idx[t, j])
            rank = seen[e]
            seen[e] += 1
            if cap is None or rank < cap:
                kept[e].append((t, j))
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + len(kept[e])
    A = int(offsets[E])
    row_of = -np.ones((T, k), dtype=np.int64)
    token_of = np.zeros(A, dtype=np.int64)
    for e in range(E):
        for i, (t, j) in enumerate(kept[e]):
            row_of[t, j] = offsets[e] + i
            token_of[offsets[e] + i] = t
    return dict(offsets=offsets, row_of=row_of, token_of=token_of, n_dropped=T * k - A)


# ------------------------------------------------------------- expert FFN
def silu(a):
    return a / (1.0 + np.exp(-a))


def dsilu(a):
    s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 + a * (1.0 - s))


def gelu(a):
    """Exact (erf) GELU."""
    return 0.5 * a * (1.0 + erf(a / math.sqrt(2.0)))


def dgelu(a):
    cdf = 0.5 * (1.0 + erf(a / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * a * a) / math.sqrt(2.0 * math.pi)
    return cdf + a * pdf


def expert_forward(X, w13, w2, act):
    """One expert's two-matrix FFN ([ETP]: up-projection w1 then down-projection
    w2). SwiGLU: H = silu(X W1^T) * (X W3^T), with w13 = [W1; W3] stacked
    [2f, d]; GELU: H = gelu(X W1^T), w13 = W1 [f, d]. Output O = H W2^T,
    w2 [d, f]. Returns (O, saved) with the pre-activations and H kept for
    the backward."""
    f = w2.shape[1]
    if act == "swiglu":
        ab = X @ w13.T
        a, b = ab[:, :f], ab[:, f:]
        H = silu(a) * b
        saved = dict(a=a, b=b, H=H)
    elif act == "gelu":
        a = X @ w13.T
        H = gelu(a)
        saved = dict(a=a, H=H)
    else:
        raise ValueError(act)
    return H @ w2.T, saved


# ------------------------------------------------------------- FP8 forward
# [Recipe] §8.1 and §9.1 list FP8 forward GEMMs with bf16 activations; §6.2
# stores experts in FP8 and widens them for use. The pages fix neither the
# FP8 format nor the scale granularity. Reading taken: OCP E4M3 codes, one
# power-of-two scale per row of each K-contiguous operand (a token row of the
# GEMM input, an output channel of the weight), chosen as the smallest power
# of two that brings the row's largest magnitude within E4M3's range.
E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Value of OCP E4M3 codes: sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent field 0 holds subnormals m/8 * 2^-6; S.1111.111 is NaN;
    there are no infinities, so the largest finite magnitude is 1.75 * 2^8."""
    c = np.asarray(codes).astype(np.int64)
    sgn = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return sgn * mag


def e4m3_encode(v):
    """Nearest E4M3 code to each value (|v| <= 448), ties to the even
    mantissa. The quantum is 2^(floor(log2|v|) - 3) in the normal range and
    2^-9 below 2^-6; |v| / quantum is exact in float64, so rounding it to the
    nearest integer (half to even) is the whole rounding step."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(v)):
        raise ValueError("e4m3_encode: input outside the finite range")
    _, ex = np.frexp(a)                   # a = mant * 2^ex, mant in [0.5, 1)
    e = np.maximum(ex - 1, -6)            # binade exponent, subnormals share -6
    q = np.exp2(e - 3.0)
    n = np.rint(a / q)                    # round half to even
    r = n * q                             # rounded magnitude (may reach 2^(e+1))
    _, ex2 = np.frexp(r)
    e2 = ex2 - 1
    normal = r >= 2.0 ** -6
    field = np.where(normal, e2 + 7, 0)
    mant = np.where(normal, r / np.exp2(e2) * 8.0 - 8.0, r / 2.0 ** -9)
    code = (field << 3) | mant.astype(np.int64)
    code = np.where(r == 0, 0, code)
    # sign-magnitude: the sign survives rounding to zero (-tiny -> 0x80)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


# The second OCP FP8 format, E5M2 (5 exponent bits, 2 mantissa bits), for the
# backward's gradient operands as an option (reading: the FP8 recipes' hybrid
# scheme, E4M3 for weights and activations and E5M2 for gradients; the pages
# name FP8 training without a format). Same power-of-two scaling rule, with
# E5M2's largest finite magnitude 57344 = 1.75 * 2^15 in place of 448.
E5M2_MAX = 57344.0


def e5m2_decode(codes):
    """Value of OCP E5M2 codes: sign bit, 5 exponent bits (bias 15), 2
    mantissa bits; exponent field 0 holds subnormals m/4 * 2^-14; field 31 is
    infinity (mantissa 0) or NaN."""
    c = np.asarray(codes).astype(np.int64)
    sgn = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = (c & 3).astype(np.float64)
    mag = np.where(e == 0, m / 4.0 * 2.0 ** -14, (1.0 + m / 4.0) * np.exp2(e - 15.0))
    mag = np.where(e == 31, np.where(c & 3 == 0, np.inf, np.nan), mag)
    return sgn * mag


def e5m2_encode(v):
    """Nearest E5M2 code to each value (|v| <= 57344), ties to the even
    mantissa: the quantum is 2^(floor(log2|v|) - 2) in the normal range and
    2^-16 below 2^-14, as in e4m3_encode."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E5M2_MAX) or np.any(np.isnan(v)):
        raise ValueError("e5m2_encode: input outside the finite range")
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -14)
    q = np.exp2(e - 2.0)
    r = np.rint(a / q) * q
    _, ex2 = np.frexp(r)
    e2 = ex2 - 1
    normal = r >= 2.0 ** -14
    field = np.where(normal, e2 + 15, 0)
    mant = np.where(normal, r / np.exp2(e2) * 4.0 - 4.0, r / 2.0 ** -16)
    code = (field << 2) | mant.astype(np.int64)
    code = np.where(r == 0, 0, code)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


FP8_FORMATS = {"e4m3": (8, e4m3_encode, e4m3_decode), "e5m2": (15, e5m2_encode, e5m2_decode)}


def fp8_row_scale_exp(amax, fmt="e4m3"):
    """Smallest integer e with amax <= M * 2^e (0 for an all-zero row), M the
    format's largest finite magnitude, 1.75 * 2^B (B = 8 for E4M3, 15 for
    E5M2). With amax = m * 2^e0, m in [1, 2), that is e0 - B when m <= 1.75
    and e0 - B + 1 otherwise: exact, no division by M."""
    B = FP8_FORMATS[fmt][0]
    amax = np.asarray(amax, dtype=np.float64)
    mant, ex = np.frexp(amax)             # amax = mant * 2^ex, mant in [0.5, 1)
    e = np.where(2.0 * mant <= 1.75, ex - 1 - B, ex - B)
    return np.where(amax == 0, 0, e).astype(np.int64)


def quantize_rows_fp8(X, fmt="e4m3"):
    """Per-row FP8 quantization: codes [n, K] uint8 and scale exponents [n]
    with X[i] ~= decode(codes[i]) * 2^e[i] (E4M3 by default, or E5M2).
    Scaling by a power of two is exact, so the only rounding is the encoder's."""
    X = np.asarray(X, dtype=np.float64)
    e = fp8_row_scale_exp(np.abs(X).max(axis=1, initial=0.0), fmt)
    codes = FP8_FORMATS[fmt][1](X * np.exp2(-e.astype(np.float64))[:, None])
    return codes, e


def dequantize_rows_fp8(codes, e, fmt="e4m3"):
    return FP8_FORMATS[fmt][2](codes) * np.exp2(np.asarray(e, dtype=np.float64))[:, None]


def round_bf16(v):
    """Round to the nearest bfloat16 value (8 significant bits), ties to even."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    q = np.exp2(np.maximum(ex - 1, -126) - 7.0)
    return np.sign(v) * np.rint(a / q) * q


def expert_forward_fp8(X, w13, w2, act):
    """expert_forward with both GEMMs on FP8 operands: X and w13 quantized per
    row, the up-projection taken exactly on their dequantized values; the
    activation H is kept in bf16 (the stored activation), and that bf16 H and
    w2 are quantized per row for the down-projection. The saved values for
    the backward are the pre-activations and H as computed here."""
    return expert_forward_fp8_wq(X, quantize_weights_fp8(w13), quantize_weights_fp8(w2), act)


def quantize_weights_fp8(w):
    """Dequantized per-row FP8 copy of a weight matrix (rows = output channels)."""
    return dequantize_rows_fp8(*quantize_rows_fp8(w))


def expert_forward_fp8_wq(X, w13d, w2d, act):
    """expert_forward_fp8 on weights already passed through quantize_weights_fp8
    (per-row quantization, so any subset of rows quantizes the same way)."""
    f = w2d.shape[1]
    Xd = dequantize_rows_fp8(*quantize_rows_fp8(X))
    pre = Xd @ w13d.T
    if act == "swiglu":
        a, b = pre[:, :f], pre[:, f:]
        H = silu(a) * b
        saved = dict(a=a, b=b, H=H)
    elif act == "gelu":
        a = pre
        H = gelu(a)
        saved = dict(a=a, H=H)
    else:
        raise ValueError(act)
    Hd = dequantize_rows_fp8(*quantize_rows_fp8(round_bf16(H)))
    return Hd @ w2d.T, saved

def expert_backward(X, w13, w2, saved, dO, act):
    """Backward of expert_forward for upstream dO [n, d].
    Returns (dX [n,d], dw13 (w13's shape), dw2 [d,f], dpre (gradient of the
    pre-activations, [n, 2f] or [n, f]))."""
    H = saved["H"]
    a = saved["a"]
    dH = dO @ w2                      # [n, f]
    if act == "swiglu":
        b = saved["b"]
        da = dH * b * dsilu(a)
        db = dH * silu(a)
        dpre = np.concatenate([da, db], axis=1)
    else:
        dpre = dH * dgelu(a)
    dX = dpre @ w13
    dw2 = dO.T @ H
    dw13 = dpre.T @ X
    return dX, dw13, dw2, dpre


# ----------------------------------------------- FP8 forward, block scales
# Finer scales for the same FP8 forward. [Recipe] §8.1/§9.1 (FP8 GEMMs, bf16
# activations) fix no granularity; one scale per row loses the small blocks of
# a row whose parts differ by many binades. Reading taken: every K-contiguous operand row is cut into blocks of
# FP8_BLOCK consecutive elements along K (the last block may be partial), and
# each block gets its own power-of-two scale, chosen by the per-row rule on the
# block's own maximum, then clipped to the 8-bit exponent scale's range
# [-127, 127] (a block whose maximum is below 448 * 2^-127 keeps 2^-127, and
# its elements round to E4M3 subnormals or zero). One scale per 32 elements
# along K is what gfx950's block-scaled matrix instruction applies.
FP8_BLOCK = 32
FP8_BLOCK_EXP_MIN, FP8_BLOCK_EXP_MAX = -127, 127


def quantize_blocks_fp8(X, block=FP8_BLOCK, fmt="e4m3"):
    """Per-block FP8 quantization of the rows of X [n, K]: codes [n, K] uint8
    and scale exponents [n, ceil(K / block)] with
    X[i, k] ~= e4m3_decode(codes[i, k]) * 2^e[i, k // block]."""
    X = np.asarray(X, dtype=np.float64)
    n, K = X.shape
    nb = -(-K // block)
    e = np.zeros((n, nb), dtype=np.int64)
    codes = np.zeros((n, K), dtype=np.uint8)
    for j in range(nb):
        blk = X[:, j * block:(j + 1) * block]
        ej = np.clip(fp8_row_scale_exp(np.abs(blk).max(axis=1, initial=0.0), fmt),
                     FP8_BLOCK_EXP_MIN, FP8_BLOCK_EXP_MAX)
        e[:, j] = ej
        codes[:, j * block:(j + 1) * block] = FP8_FORMATS[fmt][1](blk * np.exp2(-ej.astype(np.float64))[:, None])
    return codes, e


def dequantize_blocks_fp8(codes, e, block=FP8_BLOCK, fmt="e4m3"):
    e = np.asarray(e, dtype=np.float64)
    K = codes.shape[1]
    return FP8_FORMATS[fmt][2](codes) * np.repeat(np.exp2(e), block, axis=1)[:, :K]


def quantize_weights_fp8_block(w):
    """Dequantized block-scaled FP8 copy of a weight (rows = output channels,
    blocks along the input dimension)."""
    return dequantize_blocks_fp8(*quantize_blocks_fp8(w))


def expert_forward_fp8_block(X, w13, w2, act):
    """expert_forward_fp8 with block scales: X and w13 quantized per block of
    their rows, the up-projection taken exactly on the dequantized values; H
    kept in bf16, then that bf16 H and w2 quantized per block for the
    down-projection."""
    return expert_forward_fp8_block_wq(X, quantize_weights_fp8_block(w13),
                                       quantize_weights_fp8_block(w2), act)


def expert_forward_fp8_block_wq(X, w13d, w2d, act):
    """expert_forward_fp8_block on weights already passed through
    quantize_weights_fp8_block (rows quantize independently, so any subset of
    weight rows quantizes the same way)."""
    f = w2d.shape[1]
    Xd = dequantize_blocks_fp8(*quantize_blocks_fp8(X))
    pre = Xd @ w13d.T
    if act == "swiglu":
        a, b = pre[:, :f], pre[:, f:]
        H = silu(a) * b
        saved = dict(a=a, b=b, H=H)
    elif act == "gelu":
        a = pre
        H = gelu(a)
        saved = dict(a=a, H=H)
    else:
        raise ValueError(act)
    Hd = dequantize_blocks_fp8(*quantize_blocks_fp8(round_bf16(H)))
    return Hd @ w2d.T, saved


# --------------------------------------- FP8 weights in square blocks
# [Recipe] §8.1/§9.1 (FP8 training, bf16 activations) fix no granularity for
# the weights either. Reading taken for the square mode: every weight matrix
# is quantized once per step in FP8_SQUARE x FP8_SQUARE squares of the stored
# matrix (rows x columns, from its first row and column; the last ones may be
# partial), each square with one power-of-two scale chosen by the block rule
# of quantize_blocks_fp8 on the square's maximum. A square is a block along
# either dimension, so the one dequantized weight serves the forward (read
# along its input dimension) and the data gradients (read along its output
# dimension). Activations and gradients entering a GEMM keep 1 x 32 blocks
# along that GEMM's reduction axis (quantize_blocks_fp8).
FP8_SQUARE = 32


def quantize_squares_fp8(W, block=FP8_SQUARE, fmt="e4m3"):
    """Square-block FP8 quantization of W [R, C]: codes [R, C] uint8 and
    scale exponents [ceil(R / block), ceil(C / block)] with
    W[i, j] ~= decode(codes[i, j]) * 2^e[i // block, j // block]."""
    W = np.asarray(W, dtype=np.float64)
    R, C = W.shape
    nr, nc = -(-R // block), -(-C // block)
    e = np.zeros((nr, nc), dtype=np.int64)
    codes = np.zeros((R, C), dtype=np.uint8)
    for i in range(nr):
        for j in range(nc):
            rs, cs = slice(i * block, (i + 1) * block), slice(j * block, (j + 1) * block)
            sq = W[rs, cs]
            eij = int(np.clip(fp8_row_scale_exp(np.abs(sq).max(initial=0.0), fmt),
                              FP8_BLOCK_EXP_MIN, FP8_BLOCK_EXP_MAX))
            e[i, j] = eij
            codes[rs, cs] = FP8_FORMATS[fmt][1](sq * 2.0 ** -eij)
    return codes, e


def dequantize_squares_fp8(codes, e, block=FP8_SQUARE, fmt="e4m3"):
    R, C = codes.shape
    s = np.exp2(np.asarray(e, dtype=np.float64))
    s = np.repeat(np.repeat(s, block, axis=0), block, axis=1)[:R, :C]
    return FP8_FORMATS[fmt][2](codes) * s


def quantize_weights_fp8_square(w):
    """Dequantized square-block FP8 copy of a weight matrix (same shape)."""
    return dequantize_squares_fp8(*quantize_squares_fp8(w))


def expert_forward_fp8_square(X, w13, w2, act):
    """expert_forward_fp8_block with square-block weights: X and the bf16 H
    in 1 x 32 blocks along their rows, w13 and w2 in 32 x 32 squares."""
    return expert_forward_fp8_block_wq(X, quantize_weights_fp8_square(w13),
                                       quantize_weights_fp8_square(w2), act)


# ------------------------------------------------------------ FP8 backward
# [Megatron10x] §5.2 trains in FP8 mixed precision and [Recipe] §8.1/§9.1 list
# FP8 training with bf16 activations; which backward GEMMs run in FP8 is not
# stated. Reading taken: the two data-gradient GEMMs use the forward's per-row
# scheme. Their weight operand is the weight read along its input dimension,
# so it is quantized per row of its transpose (per input channel). The weight
# gradients, which reduce over tokens, stay on the unquantized values.
def quantize_weights_fp8_t(w):
    """Dequantized copy of w^T quantized per row (one scale per input channel
    of w), shape w.T: the data-gradient GEMMs' weight operand."""
    return dequantize_rows_fp8(*quantize_rows_fp8(np.asarray(w, dtype=np.float64).T))


def expert_backward_fp8_wq(X, w2td, w13td, saved, dO, act, grad_fmt="e4m3", grad_scale="row"):
    """expert_backward with its data-gradient GEMMs on FP8 operands. w2td and
    w13td come from quantize_weights_fp8_t(w2) and quantize_weights_fp8_t(w13)
    (per-row mode), or are the transposes of quantize_weights_fp8_square(w2)
    and quantize_weights_fp8_square(w13) (square mode).
    With bf16 activations, the values that reach a quantizer are the stored
    bf16 ones: dO, the saved pre-activations a (and b), and dpre. grad_fmt:
    the FP8 format of the two gradient operands (dO, dpre), E4M3 or E5M2;
    grad_scale: "row" quantizes them per row, "block" per 1 x 32 block of
    their rows (the square mode).
      dH   = deq(q(bf16 dO)) @ w2td^T
      dpre = activation backward of dH on bf16 a (and b)
      dX   = deq(q(bf16 dpre)) @ w13td^T
      dW2  = dO^T H,  dW13 = dpre^T X        (unquantized)
    Returns (dX, dw13, dw2, dpre) as expert_backward does."""
    def qg(m):
        m = round_bf16(m)
        if grad_scale == "block":
            return dequantize_blocks_fp8(*quantize_blocks_fp8(m, fmt=grad_fmt), fmt=grad_fmt)
        return dequantize_rows_fp8(*quantize_rows_fp8(m, grad_fmt), grad_fmt)
    H = saved["H"]
    a = round_bf16(saved["a"])
    dH = qg(dO) @ w2td.T
    if act == "swiglu":
        b = round_bf16(saved["b"])
        dpre = np.concatenate([dH * b * dsilu(a), dH * silu(a)], axis=1)
    else:
        dpre = dH * dgelu(a)
    dX = qg(dpre) @ w13td.T
    return dX, dpre.T @ X, dO.T @ H, dpre


# ------------------------------------------------ FP8 weight gradients
# [Megatron10x] §5.2 trains in FP8 mixed precision; the weight-gradient GEMMs
# reduce over an expert's tokens, so their operands are read along the token
# axis. Reading taken: both operands of dW2 = dO^T H and dW13 = dpre^T X are
# quantized per column with one power-of-two scale per block of 32 consecutive
# tokens of the expert (blocks start at the expert's first row; the last one
# may be partial), by the block rule of quantize_blocks_fp8 applied to the
# transposed operands; the values quantized are the stored bf16 ones.
def expert_wgrad_fp8(X, H, dO, dpre, grad_fmt="e4m3"):
    """(dW13, dW2) of one expert with FP8 block-scaled operands along the
    token axis: X [n, d], H [n, f], dO [n, d], dpre [n, 2f|f].
      dW2  = deq(qb(bf16 dO ^T)) @ deq(qb(bf16 H ^T))^T
      dW13 = deq(qb(bf16 dpre ^T)) @ deq(qb(X ^T))^T
    qb: quantize_blocks_fp8 of each row of the transposed operand (a column of
    the token-major one), blocks of 32 tokens. grad_fmt: the FP8 format of the
    gradient operands dO and dpre (X and H are E4M3)."""
    def qt(m, fmt="e4m3"):
        mt = round_bf16(np.asarray(m, dtype=np.float64)).T
        return dequantize_blocks_fp8(*quantize_blocks_fp8(mt, fmt=fmt), fmt=fmt)
    return qt(dpre, grad_fmt) @ qt(X).T, qt(dO, grad_fmt) @ qt(H).T


def grouped_ffn_forward(x_perm, offsets, w13, w2, act, x=None, sw13=None, sw2=None, fp8=False):
    """Grouped GEMM of [Recipe] §4.2: the same result as running every
    expert's GEMMs on its own contiguous rows. Optional shared experts
    ([Recipe] §2.3 / §9.1: an expert every token passes through) read all of
    x. Returns (O [A,d], Os [T,d] or None, saved). fp8=True runs every
    expert (shared ones included) through expert_forward_fp8 (per-row
    scales), fp8="block" through expert_forward_fp8_block, fp8="square"
    through expert_forward_fp8_square."""
    fwd = {"block": expert_forward_fp8_block, "square": expert_forward_fp8_square}.get(
        fp8, expert_forward_fp8 if fp8 else expert_forward)
    E = w13.shape[0]
    A = int(offsets[E])
    d = w2.shape[1]
    O = np.zeros((A, d))
    saved = []
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        o, s = fwd(x_perm[lo:hi], w13[e], w2[e], act)
        O[lo:hi] = o
        saved.append(s)
    Os, ssaved = None, []
    if sw13 is not None:
        Os = np.zeros((x.shape[0], d))
        for s in range(sw13.shape[0]):
            o, sv = fwd(x, sw13[s], sw2[s], act)
            Os += o
            ssaved.append(sv)
    return O, Os, dict(routed=saved, shared=ssaved)


def grouped_ffn_backward(x_perm, offsets, w13, w2, saved, dO, act, x=None, sw13=None,
                         sw2=None, dY=None, fp8_dgrad=False, fp8_wgrad=False, fp8_grad="e4m3"):
    """Backward of grouped_ffn_forward: per-expert dgrad and wgrad.
    The shared expert's upstream gradient is dY itself (gate 1).
    fp8_dgrad: the data gradients on FP8 operands (expert_backward_fp8_wq):
    True with per-row scales, "square" with square-block weights and 1 x 32
    block gradients.
    fp8_wgrad: the weight gradients on FP8 operands (expert_wgrad_fp8, on
    the expert's own dpre). fp8_grad: the FP8 format of the gradient operands
    of both ("e4m3" or "e5m2")."""
    E = w13.shape[0]
    dX_perm = np.zeros_like(x_perm)
    dw13 = np.zeros_like(w13)
    dw2 = np.zeros_like(w2)
    dpre_r = np.zeros((x_perm.shape[0], w13.shape[1]))

    def bwd(X, w13e, w2e, sv, g):
        if fp8_dgrad == "square":
            out = expert_backward_fp8_wq(X, quantize_weights_fp8_square(w2e).T,
                                         quantize_weights_fp8_square(w13e).T, sv, g, act, fp8_grad,
                                         "block")
        elif fp8_dgrad:
            out = expert_backward_fp8_wq(X, quantize_weights_fp8_t(w2e),
                                         quantize_weights_fp8_t(w13e), sv, g, act, fp8_grad)
        else:
            out = expert_backward(X, w13e, w2e, sv, g, act)
        if fp8_wgrad:
            dx, _, _, dp = out
            g13, g2 = expert_wgrad_fp8(X, sv["H"], g, dp, fp8_grad)
            out = (dx, g13, g2, dp)
        return out

    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        dx, g13, g2, dp = bwd(x_perm[lo:hi], w13[e], w2[e], saved["routed"][e], dO[lo:hi])
        dX_perm[lo:hi] = dx
        dpre_r[lo:hi] = dp
        dw13[e] = g13
        dw2[e] = g2
    dXs = dsw13 = dsw2 = dpre_s = None
    if sw13 is not None:
        dXs = np.zeros_like(x)
        dsw13 = np.zeros_like(sw13)
        dsw2 = np.zeros_like(sw2)
        for s in range(sw13.shape[0]):
            dx, g13, g2, dpre_s = bwd(x, sw13[s], sw2[s], saved["shared"][s], dY)
            dXs += dx
            dsw13[s] = g13
            dsw2[s] = g2
    # dpre: gradient of the pre-activations per routed row (and of the last shared expert)
    return dict(dx_perm=dX_perm, dw13=dw13, dw2=dw2, dx_shared=dXs, dsw13=dsw13, dsw2=dsw2,
                dpre=dpre_r, dpre_shared=dpre_s)


# ----------------------------------------------------------------- combine
def combine(O, gates, row_of, Os=None):
    """Weighted sum of [Recipe] §2.1/§2.2: Y[t] = Os[t] + sum over kept slots
    j of g_tj * O[row(t,j)]. A dropped slot adds nothing (no renormalisation)."""
    T, k = row_of.shape
    Y = np.zeros((T, O.shape[1])) if Os is None else Os.copy()
    for t in range(T):
        for j in range(k):
            r = row_of[t, j]
            if r >= 0:
                Y[t] += gates[t, j] * O[r]
    return Y


def combine_backward(dY, O, gates, row_of):
    """dgate_tj = <dY[t], O[row(t,j)]> (0 if dropped); dO[row(t,j)] = g_tj dY[t]."""
    T, k = row_of.shape
    dgate = np.zeros((T, k))
    dO = np.zeros_like(O)
    for t in range(T):
        for j in range(k):
            r = row_of[t, j]
            if r >= 0:
                dgate[t, j] = float(dY[t] @ O[r])
                dO[r] = gates[t, j] * dY[t]
    return dgate, dO


# ---------------------------------------------------------- router backward
def router_backward(x, w_r, scores, topk_idx, gates, dgate, score="softmax", aux_coef=0.0,
                    y=None, z_coef=0.0, logits=None, tau=None, n_tokens=None):
    """Gradient of the router through the renormalised gates of [Recipe] §2.2
    (the top-k choice itself is piecewise constant), plus aux_coef times the
    gradient of L_aux = E sum_i y_i z_i with the counts y held fixed.

    Softmax: the renormalised gates equal a softmax over the chosen logits,
      dl_e = g_e (dg_e - sum_j g_j dg_j) for chosen e, 0 otherwise.
    Sigmoid: g_j = s_j / sum_S s,
      dl_e = s_e (1 - s_e) (dg_e - sum_j g_j dg_j) / sum_S s for chosen e.
    Aux (z_i = mean_t s_ti):
      softmax: dl_te += aux_coef (E/T) s_te (y_e - sum_i y_i s_ti)
      sigmoid: dl_te += aux_coef (E/T) y_e s_te (1 - s_te)
    Plus z_coef times the gradient of z_loss(logits) when z_coef != 0.
    With the noisy gate (tau given) these are gradients with respect to the
    noisy logits (l + g) / tau; the chain rule to l divides them by tau.
    Returns dict(dlogits [T,E], dw_r [E,d] = dl^T x, dx_router [T,d] = dl W_r),
    dlogits being the gradient with respect to l.
    n_tokens: the batch's token count in the 1/T factors of the aux and z-loss
    terms when the rows given are a subset of the batch (default: all rows).
    """
    T, E = scores.shape
    if n_tokens is not None:
        T = n_tokens
    k = topk_idx.shape[1]
    dl = np.zeros(scores.shape)
    for t in range(scores.shape[0]):
        sel = topk_idx[t]
        g = gates[t]
        dg = dgate[t]
        inner = float((g * dg).sum())
        if score == "softmax":
            dl[t, sel] = g * (dg - inner)
        else:
            s = scores[t, sel]
            dl[t, sel] = s * (1.0 - s) * (dg - inner) / s.sum()
    if aux_coef != 0.0:
        if score == "softmax":
            ys = scores @ y
            dl += aux_coef * (E / T) * scores * (y[None, :] - ys[:, None])
        else:
            dl += aux_coef * (E / T) * y[None, :] * scores * (1.0 - scores)
    if z_coef != 0.0:
        dl += z_coef * z_loss_grad(logits, T)
    if tau is not None:
        dl = dl / tau
    return dict(dlogits=dl, dw_r=dl.T @ x, dx_router=dl @ w_r)


# ------------------------------------------- aux-loss-free bias, z-loss
def bias_update(bias, counts, T, k, gamma):
    """Aux-loss-free balancing of [Recipe] §5.3/§5.4: with the load f_i of
    expert i (here y_i = counts_i / (T k)) and target 1/E,
    b_i <- b_i + gamma * sign(1/E - f_i); an exactly balanced expert keeps b_i.
    The comparison f_i < 1/E is made exactly as counts_i * E < T * k."""
    E = bias.shape[0]
    load = np.asarray(counts, dtype=np.int64) * E
    target = T * k
    step = np.where(load < target, 1.0, np.where(load > target, -1.0, 0.0))
    return bias + gamma * step


def router_logsumexp(logits):
    """log sum_e exp(l_te) per token (max-subtracted)."""
    m = logits.max(axis=1)
    return m + np.log(np.exp(logits - m[:, None]).sum(axis=1))


def z_loss(logits):
    """Router z-loss, named by [Recipe] §9.1/§9.2 with weight 1e-3 but without a
    formula on the pages; read as mean_t (logsumexp_e l_te)^2 (the common
    definition). Gradient: d/dl_te = (2/T) lse_t softmax(l_t)_e."""
    lse = router_logsumexp(logits)
    return float(np.mean(lse * lse))


def z_loss_grad(logits, n_tokens=None):
    T = logits.shape[0] if n_tokens is None else n_tokens
    lse = router_logsumexp(logits)
    sm = np.exp(logits - lse[:, None])
    return (2.0 / T) * lse[:, None] * sm


def permute_backward(dx_perm, row_of, dx_shared=None, dx_router=None):
    """Un-permute: dX[t] = dXs[t] + sum over kept j of dX_perm[row(t,j)] + dx_router[t]."""
    T, k = row_of.shape
    dX = np.zeros((T, dx_perm.shape[1]))
    if dx_shared is not None:
        dX += dx_shared
    for t in range(T):
        for j in range(k):
            r = row_of[t, j]
            if r >= 0:
                dX[t] += dx_perm[r]
    if dx_router is not None:
        dX += dx_router
    return dX


# ------------------------------------------------------------- whole layer
def layer_forward(x, w_r, w13, w2, k, score="softmax", act="swiglu", cap=None,
                  logit_bias=None, sel_bias=None, sw13=None, sw2=None, gumbel_u=None, tau=None,
                  fp8=False):
    """Forward of the layer: router, stats, permute, grouped FFN, combine.
    All arrays float64 (exact values of the fp32/bf16 inputs)."""
    E = w13.shape[0]
    r = router_forward(x, w_r, k, score, logit_bias, sel_bias, gumbel_u, tau)
    st = aux_stats(r["scores"], r["topk_idx"], E)
    p = permute(r["topk_idx"], E, cap)
    x_perm = x[p["token_of"]]
    O, Os, saved = grouped_ffn_forward(x_perm, p["offsets"], w13, w2, act, x, sw13, sw2, fp8)
    Y = combine(O, r["gates"], p["row_of"], Os)
    return dict(router=r, stats=st, perm=p, x_perm=x_perm, O=O, Os=Os, saved=saved, Y=Y)


def layer_backward(fwd, x, w_r, w13, w2, dY, score="softmax", act="swiglu", aux_coef=0.0,
                   sw13=None, sw2=None, z_coef=0.0, tau=None, fp8_dgrad=False, fp8_wgrad=False,
                   fp8_grad="e4m3"):
    """Backward of the layer for upstream dY: combine bwd, grouped FFN bwd,
    router bwd, un-permute."""
    r, p = fwd["router"], fwd["perm"]
    dgate, dO = combine_backward(dY, fwd["O"], r["gates"], p["row_of"])
    g = grouped_ffn_backward(fwd["x_perm"], p["offsets"], w13, w2, fwd["saved"], dO, act, x,
                             sw13, sw2, dY, fp8_dgrad, fp8_wgrad, fp8_grad)
    rb = router_backward(x, w_r, r["scores"], r["topk_idx"], r["gates"], dgate, score,
                         aux_coef, fwd["stats"]["y"], z_coef, r["logits"], tau)
    dX = permute_backward(g["dx_perm"], p["row_of"], g["dx_shared"], rb["dx_router"])
    return dict(dgate=dgate, dO=dO, dX=dX, **g, **rb)
