"""Mutation check of the oracle's pins: each case plants one plausible mistake
in a copy of the oracle's source (a dropped renormalisation, a wrong sign, a
wrong index, an off-by-one comparison ...) and runs the pins that should
catch it against the mutant. Every mutant must fail at least one of them;
a mutant that passes means the pins have a blind spot.

The mutants are built from oracle/moe_oracle.py's text on the CPU; the real
oracle module is never modified. Each planted change must match the source
exactly once, so a later edit of the oracle cannot make a case vacuous.
"""
import os
import types

import numpy as np
import pytest

import test_oracle_pins as P

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "moe_oracle.py")
with open(SRC_PATH, encoding="utf-8") as _fh:
    SRC = _fh.read()


def _mutant(old, new):
    assert SRC.count(old) == 1, f"planted change does not match the oracle exactly once: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _fails(mod, pin, *args):
    """True when the pin raises on the mutant (the real oracle passes it:
    the same pins run unmutated in test_oracle_pins)."""
    saved = P.O
    P.O = mod
    try:
        pin(*[dict(a) if isinstance(a, dict) else a for a in args])
    except Exception:
        return True
    finally:
        P.O = saved
    return False


SWIGLU_FD = P.FD_VARIANTS[0]
AUX_FD = P.FD_VARIANTS[1]
SIGMOID_FD = P.FD_VARIANTS[3]

# (name, old text, new text, pins expected to catch it)
MUTANTS = [
    ("gates not renormalised",
     "gates = chosen / chosen.sum(axis=1, keepdims=True)", "gates = chosen",
     [(P.test_zero_router_weight_tie_break_and_stats,),
      (P.test_sparse_oracle_equals_dense_brute_force, P.VARIANTS[0])]),
    ("ties to the higher expert index",
     'order = np.argsort(-key, axis=1, kind="stable")',
     'order = key.shape[1] - 1 - np.argsort(-key[:, ::-1], axis=1, kind="stable")',
     [(P.test_zero_router_weight_tie_break_and_stats,)]),
    ("sigmoid scores replaced by softmax",
     "scores = 1.0 / (1.0 + np.exp(-logits))",
     "scores = np.exp(logits) / np.exp(logits).sum(axis=1, keepdims=True)",
     [(P.test_sparse_oracle_equals_dense_brute_force, P.VARIANTS[4])]),
    ("selection bias also shifts the gates",
     "chosen = np.take_along_axis(scores, topk_idx, axis=1)",
     "chosen = np.take_along_axis(key, topk_idx, axis=1)",
     [(P.test_sparse_oracle_equals_dense_brute_force, P.VARIANTS[4])]),
    ("y normalised by T instead of T k",
     "y = counts / float(T * k)", "y = counts / float(T)",
     [(P.test_hand_computed_aux_stats,), (P.test_golden_uniform_top2_ratio,),
      (P.test_zero_router_weight_tie_break_and_stats,)]),
    ("z taken over the chosen experts only",
     "z = scores.mean(axis=0)",
     "z = (scores * (np.arange(E)[None, :] == topk_idx[:, :1])).mean(axis=0)",
     [(P.test_hand_computed_aux_stats,), (P.test_zero_router_weight_tie_break_and_stats,)]),
    ("capacity rounded down",
     "return int(math.ceil(cf * T * k / E))", "return int(math.floor(cf * T * k / E))",
     [(P.test_golden_capacity_worked_example,), (P.test_capacity_rounds_up_a_fractional_limit,)]),
    ("capacity test off by one (<=)",
     "if cap is None or rank < cap:", "if cap is None or rank <= cap:",
     [(P.test_capacity_keeps_first_tokens_when_all_go_to_one_expert,),
      (P.test_capacity_zero_drops_everything,),
      (P.test_sparse_oracle_equals_dense_brute_force, P.VARIANTS[2])]),
    ("gates renormalised over the kept slots after a drop",
     "                Y[t] += gates[t, j] * O[r]",
     "                Y[t] += gates[t, j] / gates[t][row_of[t] >= 0].sum() * O[r]",
     [(P.test_sparse_oracle_equals_dense_brute_force, P.VARIANTS[2])]),
    ("wrong sign in silu'",
     "return s * (1.0 + a * (1.0 - s))", "return s * (1.0 - a * (1.0 - s))",
     [(P.test_activation_derivatives,), (P.test_gradients_by_central_differences, SWIGLU_FD)]),
    ("tanh GELU instead of the erf form",
     "return 0.5 * a * (1.0 + erf(a / math.sqrt(2.0)))",
     "return 0.5 * a * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (a + 0.044715 * a ** 3)))",
     [(P.test_activation_derivatives,), (P.test_single_expert_is_textbook_ffn, "gelu")]),
    ("gate and up halves swapped",
     "a, b = ab[:, :f], ab[:, f:]", "b, a = ab[:, :f], ab[:, f:]",
     [(P.test_single_expert_is_textbook_ffn, "swiglu"),
      (P.test_sparse_oracle_equals_dense_brute_force, P.VARIANTS[0])]),
    ("down-matrix weight gradient from the pre-activation instead of H",
     "    dw2 = dO.T @ H\n", "    dw2 = dO.T @ a\n",
     [(P.test_gradients_by_central_differences, SWIGLU_FD)]),
    ("first-matrix weight gradient from the upstream gradient's rows in reverse",
     "    dw13 = dpre.T @ X\n", "    dw13 = dpre.T @ X[::-1]\n",
     [(P.test_gradients_by_central_differences, SWIGLU_FD)]),
    ("dgate from the wrong slot's row",
     "dgate[t, j] = float(dY[t] @ O[r])", "dgate[t, j] = float(dY[t] @ O[row_of[t, 0]])",
     [(P.test_gradients_by_central_differences, SWIGLU_FD)]),
    ("aux gradient dropped",
     "dl += aux_coef * (E / T) * scores * (y[None, :] - ys[:, None])", "dl += 0.0",
     [(P.test_aux_gradient_is_not_dropped,), (P.test_gradients_by_central_differences, AUX_FD)]),
    ("sigmoid router gradient without the 1/sum denominator",
     "dl[t, sel] = s * (1.0 - s) * (dg - inner) / s.sum()",
     "dl[t, sel] = s * (1.0 - s) * (dg - inner)",
     [(P.test_gradients_by_central_differences, SIGMOID_FD)]),
    ("noisy-gate chain factor multiplies by tau",
     "dl = dl / tau", "dl = dl * tau",
     [(P.test_layer_gradient_with_noisy_gate_by_central_differences,)]),
    ("Gumbel noise with the wrong sign",
     "return -np.log(-np.log(u + GUMBEL_EPS) + GUMBEL_EPS)",
     "return np.log(-np.log(u + GUMBEL_EPS) + GUMBEL_EPS)",
     [(P.test_gumbel_noise_hand_values,), (P.test_gumbel_max_samples_the_softmax,)]),
    ("z-loss without the square",
     "return float(np.mean(lse * lse))", "return float(np.mean(lse))",
     [(P.test_z_loss_closed_form_and_gradient,)]),
    ("bias update pushes the wrong way",
     "step = np.where(load < target, 1.0, np.where(load > target, -1.0, 0.0))",
     "step = np.where(load < target, -1.0, np.where(load > target, 1.0, 0.0))",
     [(P.test_bias_update_rule,), (P.test_bias_update_balances_a_skewed_router,)]),
    ("un-permute drops the router's term",
     "    if dx_router is not None:\n        dX += dx_router\n", "",
     [(P.test_gradients_by_central_differences, SWIGLU_FD)]),
    ("E4M3 rounding half away from zero instead of to even",
     "n = np.rint(a / q)                    # round half to even",
     "n = np.floor(a / q + 0.5)",
     [(P.test_e4m3_encode_matches_library_rounding,)]),
    ("FP8 scale exponent one too large at the boundary mantissa",
     "e = np.where(2.0 * mant <= 1.75, ex - 1 - B, ex - B)",
     "e = np.where(2.0 * mant < 1.75, ex - 1 - B, ex - B)",
     [(P.test_fp8_row_scale_is_the_smallest_power_of_two,)]),
    ("data-gradient weights scaled per output channel instead of per input channel",
     "return dequantize_rows_fp8(*quantize_rows_fp8(np.asarray(w, dtype=np.float64).T))",
     "return dequantize_rows_fp8(*quantize_rows_fp8(np.asarray(w, dtype=np.float64))).T",
     [(P.test_expert_backward_fp8_exact_with_per_channel_scales,)]),
    ("FP8 down-projection quantizes H without its bf16 rounding",
     "Hd = dequantize_rows_fp8(*quantize_rows_fp8(round_bf16(H)))",
     "Hd = dequantize_rows_fp8(*quantize_rows_fp8(H))",
     [(P.test_expert_forward_fp8_brute_force, "swiglu")]),
    ("FP8 block scales: one scale per row instead of per block",
     "ej = np.clip(fp8_row_scale_exp(np.abs(blk).max(axis=1, initial=0.0), fmt),",
     "ej = np.clip(fp8_row_scale_exp(np.abs(X).max(axis=1, initial=0.0), fmt),",
     [(P.test_fp8_blocks_keep_small_blocks_that_a_row_scale_loses,),
      (P.test_fp8_blocks_brute_force_and_partial_last_block,)]),
    ("FP8 block exponent not clipped to the scale range",
     "FP8_BLOCK_EXP_MIN, FP8_BLOCK_EXP_MAX = -127, 127",
     "FP8_BLOCK_EXP_MIN, FP8_BLOCK_EXP_MAX = -1000, 1000",
     [(P.test_fp8_block_exponent_is_clipped_to_the_scale_range,)]),
    ("FP8 weight gradients: blocks along each token row instead of along the token axis",
     "mt = round_bf16(np.asarray(m, dtype=np.float64)).T",
     "mt = round_bf16(np.asarray(m, dtype=np.float64))",
     [(P.test_expert_wgrad_fp8_brute_force,), (P.test_fp8_wgrad_exact_on_block_exact_columns,)]),
    ("FP8 weight gradients quantize dpre without its bf16 rounding",
     "mt = round_bf16(np.asarray(m, dtype=np.float64)).T",
     "mt = np.asarray(m, dtype=np.float64).T",
     [(P.test_expert_wgrad_fp8_brute_force,)]),
    ("E5M2 scale taken with E4M3's largest magnitude",
     'FP8_FORMATS = {"e4m3": (8, e4m3_encode, e4m3_decode), "e5m2": (15, e5m2_encode, e5m2_decode)}',
     'FP8_FORMATS = {"e4m3": (8, e4m3_encode, e4m3_decode), "e5m2": (8, e5m2_encode, e5m2_decode)}',
     [(P.test_e5m2_row_scale_is_the_smallest_power_of_two,)]),
    ("FP8 weight gradients quantize dO in E4M3 whatever the gradient format",
     "return qt(dpre, grad_fmt) @ qt(X).T, qt(dO, grad_fmt) @ qt(H).T",
     "return qt(dpre, grad_fmt) @ qt(X).T, qt(dO) @ qt(H).T",
     [(P.test_expert_wgrad_fp8_e5m2_gradients_brute_force,)]),
    ("FP8 squares: each row of a square scaled on its own",
     "eij = int(np.clip(fp8_row_scale_exp(np.abs(sq).max(initial=0.0), fmt),",
     "eij = int(np.clip(fp8_row_scale_exp(np.abs(sq[:1]).max(initial=0.0), fmt),",
     [(P.test_fp8_squares_brute_force_with_partial_edges,),
      (P.test_fp8_squares_share_one_scale_down_the_rows,)]),
    ("FP8 squares: exponents laid out transposed",
     "s = np.repeat(np.repeat(s, block, axis=0), block, axis=1)[:R, :C]",
     "s = np.repeat(np.repeat(s.T, block, axis=0), block, axis=1)[:R, :C]",
     [(P.test_fp8_squares_brute_force_with_partial_edges,)]),
    ("square-mode data gradients quantize the gradients per row",
     'if grad_scale == "block":', 'if grad_scale == "blocks":',
     [(P.test_expert_backward_fp8_square_brute_force, "swiglu", False)]),
    ("square-mode data gradients read the weights along their input dimension",
     "out = expert_backward_fp8_wq(X, quantize_weights_fp8_square(w2e).T,",
     "out = expert_backward_fp8_wq(X, quantize_weights_fp8_t(w2e),",
     [(P.test_grouped_square_mode_is_per_expert,)]),
]


@pytest.mark.parametrize("name,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(name, old, new, pins):
    mod = _mutant(old, new)
    caught = [pin[0].__name__ for pin in pins if _fails(mod, *pin)]
    assert caught, f"mutant '{name}' passes every pin it was meant to fail"


def test_unmutated_copy_passes_the_same_pins():
    """The harness itself: a copy built from the unchanged source passes
    every pin used above (so a failure above is the mutation's doing)."""
    mod = types.ModuleType("oracle_copy")
    exec(compile(SRC, "oracle_copy", "exec"), mod.__dict__)
    seen = set()
    for _, _, _, pins in MUTANTS:
        for pin in pins:
            key = (pin[0].__name__, repr(pin[1:]))
            if key in seen:
                continue
            seen.add(key)
            assert not _fails(mod, *pin), f"unmutated copy fails {pin[0].__name__}"
