"""The seeded workloads have the load shapes their descriptions state,
measured with the oracle's router on the committed draws (CPU only).

Skewed load: experts 0 and 3 take about two thirds of the assignments
([Megatron10x] §2.1 reports 68% on two experts) and experts 5 and 6 under 3%
each, with and without the capacity limit (the limit acts after routing).
"""
import numpy as np
import pytest

import oracle as O
from moe_inputs import WORKLOADS, as_f64, gen_logit_bias, gen_router_weight, gen_x


@pytest.mark.parametrize("name", ["skewed_bf16", "skewed_nocap_bf16", "skewed_cf15_bf16"])
def test_skewed_expert_shares(name):
    w = WORKLOADS[name]
    x = as_f64(gen_x(w), w.dtype)
    r = O.router_forward(x, gen_router_weight(w).astype(np.float64), w.k, w.score,
                         gen_logit_bias(w).astype(np.float64))
    y = O.aux_stats(r["scores"], r["topk_idx"], w.E)["y"]
    assert 0.64 <= y[0] + y[3] <= 0.72, y
    assert y[5] < 0.03 and y[6] < 0.03, y
    # the cold experts still receive tokens: their GEMM groups are small, not empty
    assert y[5] * w.T * w.k > 64 and y[6] * w.T * w.k > 64, y


def test_deepseek_like_loads():
    """256 experts at top-8 over 8192 tokens: a mean of 256 rows per expert,
    spread roughly 150-420 (the small groups the grouped GEMM must serve)."""
    w = WORKLOADS["dsv3_bf16"].replace(T=2048)
    x = as_f64(gen_x(w), w.dtype)
    from moe_inputs import gen_sel_bias
    r = O.router_forward(x, gen_router_weight(w).astype(np.float64), w.k, w.score, None,
                         gen_sel_bias(w).astype(np.float64))
    c = O.aux_stats(r["scores"], r["topk_idx"], w.E)["counts"]
    assert c.sum() == w.T * w.k
    assert c.min() > 0 and c.max() < 3 * c.mean()
