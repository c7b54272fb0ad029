"""Where the FP8 parity bounds come from, computed on the CPU.

Both sides quantize a bf16 tensor that each computes itself: H (the FP8
forward's activation, quantized for the down-projection) and dpre (the FP8
data gradient's pre-activation gradient, quantized for dX). The device
computes the values before that rounding in float32 on the matrix cores, the
oracle in float64. Where the two land on different sides of an E4M3 rounding
boundary, the quantized codes differ by one E4M3 step (2^-4 to 2^-3 of the
element) and the next product moves by much more than bf16 rounding.

How far: one flipped code of H_j moves O[i, c] by up to 2^-3 |H_j| |W2[c, j]|,
with |W2| up to about 4.5 / sqrt(f) (normal weights of std 1/sqrt(f)) and
|H_j| up to about 3 rms(H), against max|O| of about 4 rms(O) = 4 rms(H); so
about 2^-3 * 3 * 4.5 / 4 / sqrt(f) = 0.42 / sqrt(f) of max|O|. dX from a
flipped dpre code is bounded the same way (0.5 / sqrt(f) covers both). The
GPU parity tests therefore hold
  FP8 forward, O:        max|d| <= max(2e-2, 0.5 / sqrt(f)) max|ref|
  FP8 data gradient, dX: max|d| <= max(5e-2, 0.5 / sqrt(f)) max|ref|, L1 <= 1.5e-2
(tests/parity_util.py: fp8_fwd_tol, fp8_dgrad_tol).

This file emulates the device's arithmetic on the oracle's operands: float32
products and sums plus the matrix cores' accumulation error (normal, std
ACC_SIGMA of each 64-k instruction's sum|products|; measured on gfx950 with
an FP8 GEMM on the same matrix cores: median 1.2e-6, 99th percentile 9.5e-6
of sum|products| for K = 64, which ACC_SIGMA over-covers about threefold, see
test_gpu_fp8_accum.py), float32 activation maths, bf16 rounding, then the
oracle's own E4M3 quantizer. It measures how far the routed output of several
experts lands from the oracle's, at the shapes of the GPU parity tests, and
checks the bounds hold with margin and are not loose by orders of magnitude.
"""
import numpy as np
import pytest

import oracle as O
from moe_inputs import bf16_bits_to_f32, to_bf16_bits
from parity_util import fp8_dgrad_tol, fp8_fwd_tol

ACC_SIGMA = 5e-6   # accumulation error per matrix-core instruction: normal, std relative to sum|products|


def _bf16(v):
    """float32 values rounded to bf16 (round to nearest even), as float64."""
    return bf16_bits_to_f32(to_bf16_bits(np.asarray(v, dtype=np.float32))).astype(np.float64)


def _device_matmul(A, B, rng):
    """A @ B.T of exactly representable operands as the device takes it:
    float32 products and sums, plus, for each 64-k instruction, an
    accumulation error drawn from a normal of std ACC_SIGMA times that
    instruction's sum|products| (independent per instruction and element)."""
    out = np.asarray(A, np.float32) @ np.asarray(B, np.float32).T
    out = out.astype(np.float64)
    for k0 in range(0, A.shape[1], 64):
        scale = np.abs(A[:, k0:k0 + 64]) @ np.abs(B[:, k0:k0 + 64]).T
        out += rng.standard_normal(out.shape) * ACC_SIGMA * scale
    return out


def _silu32(a):
    a = np.asarray(a, np.float32)
    return a / (np.float32(1.0) + np.exp(-a))


def _dsilu32(a):
    a = np.asarray(a, np.float32)
    s = np.float32(1.0) / (np.float32(1.0) + np.exp(-a))
    return s * (np.float32(1.0) + a * (np.float32(1.0) - s))


def _draw(rng, n, d, f):
    X = _bf16(rng.standard_normal((n, d)))
    w13 = _bf16(rng.standard_normal((2 * f, d)) / np.sqrt(d))
    w2 = _bf16(rng.standard_normal((d, f)) / np.sqrt(f))
    return X, w13, w2


def _rel(got, ref):
    err = np.abs(got - ref)
    return err.max() / np.abs(ref).max(), err.sum() / np.abs(ref).sum()


def _q_rows(m):
    return O.dequantize_rows_fp8(*O.quantize_rows_fp8(m))


def _q_blocks(m):
    return O.dequantize_blocks_fp8(*O.quantize_blocks_fp8(m))


def forward_gap(rng, E, n, d, f, block=False, square=False):
    """max and L1 relative gap of the routed O (E experts of n rows) between
    the device emulation and the oracle's FP8 forward (per-row scales, or
    one scale per 32 elements along K with block=True, and 32 x 32 weight
    squares with square=True)."""
    q, qw = (_q_blocks, O.quantize_weights_fp8_block) if block else (_q_rows, O.quantize_weights_fp8)
    if square:
        q, qw = _q_blocks, O.quantize_weights_fp8_square
    efwd = O.expert_forward_fp8_block_wq if block or square else O.expert_forward_fp8_wq
    got, ref = [], []
    for _ in range(E):
        X, w13, w2 = _draw(rng, n, d, f)
        w13d, w2d = qw(w13), qw(w2)
        r, _ = efwd(X, w13d, w2d, "swiglu")
        pre = _device_matmul(q(X), w13d, rng).astype(np.float32)
        H = _bf16(_silu32(pre[:, :f]) * pre[:, f:])
        got.append(q(H) @ w2d.T)
        ref.append(r)
    return _rel(np.concatenate(got), np.concatenate(ref))


def dgrad_gap(rng, E, n, d, f, fmt="e4m3", square=False):
    """max and L1 relative gap of dX (FP8 data gradients, E experts of n rows)
    between the device emulation and the oracle, on the oracle's own saved
    pre-activations (per-row scales, or with square=True 32 x 32 weight squares
    and 1 x 32 gradient blocks)."""
    def qg(m):
        if square:
            return O.dequantize_blocks_fp8(*O.quantize_blocks_fp8(m, fmt=fmt), fmt=fmt)
        return O.dequantize_rows_fp8(*O.quantize_rows_fp8(m, fmt), fmt)
    got, ref = [], []
    for _ in range(E):
        X, w13, w2 = _draw(rng, n, d, f)
        dO = _bf16(rng.standard_normal((n, d)))
        _, saved = O.expert_forward(X, w13, w2, "swiglu")
        if square:
            w2t, w13t = O.quantize_weights_fp8_square(w2).T, O.quantize_weights_fp8_square(w13).T
        else:
            w2t, w13t = O.quantize_weights_fp8_t(w2), O.quantize_weights_fp8_t(w13)
        r, _, _, _ = O.expert_backward_fp8_wq(X, w2t, w13t, saved, dO, "swiglu", fmt,
                                              "block" if square else "row")
        a = _bf16(saved["a"]).astype(np.float32)
        b = _bf16(saved["b"]).astype(np.float32)
        dH = _device_matmul(qg(dO), w2t, rng).astype(np.float32)
        dpre = _bf16(np.concatenate([dH * b * _dsilu32(a), dH * _silu32(a)], axis=1))
        got.append(qg(dpre) @ w13t.T)
        ref.append(r)
    return _rel(np.concatenate(got), np.concatenate(ref))


# (experts, rows per expert, d, f): the reduced FP8 layers of the GPU tests
# (DeepSeek-like: 32 rows per expert, d 512, f 256; Mixtral-like smoke:
# d 256, f 512) and small-f shapes where a flip weighs most
SHAPES = [(32, 32, 512, 256), (8, 64, 256, 512), (16, 64, 256, 64), (8, 128, 128, 16),
          (4, 256, 256, 1024)]
SEEDS = 3


@pytest.mark.parametrize("kind", ["forward", "forward_block", "forward_square", "dgrad", "dgrad_e5m2",
                                  "dgrad_square", "dgrad_square_e5m2"])
def test_fp8_bounds_cover_the_emulated_device(kind):
    """The block- and square-scaled modes are held to the per-row bounds: a
    flipped code is one E4M3 step of its element whatever the scale's
    granularity, so the same reasoning gives the same bound."""
    gap = {"forward": forward_gap, "dgrad": dgrad_gap,
           "forward_block": lambda *a: forward_gap(*a, block=True),
           "forward_square": lambda *a: forward_gap(*a, square=True),
           "dgrad_e5m2": lambda *a: dgrad_gap(*a, fmt="e5m2"),
           "dgrad_square": lambda *a: dgrad_gap(*a, square=True),
           "dgrad_square_e5m2": lambda *a: dgrad_gap(*a, fmt="e5m2", square=True)}[kind]
    ratios = []
    for E, n, d, f in SHAPES:
        tol = fp8_dgrad_tol(f, "e5m2" if kind.endswith("e5m2") else "e4m3") if kind.startswith("dgrad") \
            else fp8_fwd_tol(f)
        l1_bound = tol.get("l1_rel", 5e-3)
        for s in range(SEEDS):
            mx, l1 = gap(np.random.default_rng(1000 + s), E, n, d, f)
            assert mx <= 0.9 * tol["max_rel"], (kind, E, n, d, f, s, mx, tol)
            assert l1 <= 0.5 * l1_bound, (kind, E, n, d, f, s, l1, l1_bound)
            ratios.append(mx / tol["max_rel"])
    # the bound is tight where flips weigh most, not loose by orders of magnitude
    assert max(ratios) > 0.3, ratios


def test_block_scaled_inputs_tell_block_from_row_scales():
    """The GPU test on block-varied inputs (x's 32-column blocks scaled by 2^s,
    s in [-10, 10], w13's input columns by 2^-s, w2's blocks by 2^r, r in
    [-4, 4]) separates a correct block-scaled forward from a per-row one and
    from block scales applied one block off: both land well outside the FP8
    forward bound."""
    rng = np.random.default_rng(7)
    n, d, f = 64, 384, 512
    X, w13, w2 = _draw(rng, n, d, f)
    col = lambda s: np.repeat(s, 32)   # noqa: E731
    sx = col(np.exp2(rng.integers(-10, 11, d // 32)))
    X, w13 = X * sx, w13 / sx
    w2 = w2 * col(np.exp2(rng.integers(-4, 5, f // 32)))
    ref, _ = O.expert_forward_fp8_block(X, w13, w2, "swiglu")
    row, _ = O.expert_forward_fp8(X, w13, w2, "swiglu")

    def shifted(m):   # each block decoded with its right neighbour's scale
        c, e = O.quantize_blocks_fp8(m)
        return O.dequantize_blocks_fp8(c, np.roll(e, -1, axis=1))
    pre = shifted(X) @ shifted(w13).T
    H = O.round_bf16(O.silu(pre[:, :f]) * pre[:, f:])
    off = shifted(H) @ shifted(w2).T
    tol = fp8_fwd_tol(f)["max_rel"]
    assert _rel(row, ref)[0] > 3 * tol
    assert _rel(off, ref)[0] > 3 * tol
