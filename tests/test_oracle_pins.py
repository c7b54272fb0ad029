"""Pins of the CPU oracle against things other than itself.

* a dense brute force (every expert run on every token, then masked by an
  independently computed routing and weighted by closed-form gates);
* closed forms (zero router weight, k = E, E = k = 1 textbook FFN via torch,
  identical experts, shared expert alone);
* invariants (gates sum to 1, counts sum to T k, permutation bijection,
  un-permute of permute);
* the worked capacity example and the uniform top-2 ratio printed on the
  pages (tests/golden);
* central finite differences of a scalar loss for every gradient.
"""
import math
import os

import numpy as np
import pytest
import scipy.special as sps
import scipy.stats as sst
import torch

import oracle as O
from moe_inputs import Workload, gen_all, as_f64, to_bf16_bits, bf16_bits_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _tiny(T=24, d=16, E=6, k=2, f=12, **kw):
    w = Workload("t", T=T, d=d, E=E, k=k, f=f, dtype="fp32", **kw)
    g = gen_all(w)
    conv = {n: as_f64(v, w.dtype) for n, v in g.items()}
    return w, conv


# --------------------------------------------------------------- brute force
def _brute_select(key, k):
    """Per token: repeatedly take the largest key, lowest index on equal keys."""
    T, E = key.shape
    idx = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        remaining = list(range(E))
        for j in range(k):
            best = remaining[0]
            for e in remaining[1:]:
                if key[t, e] > key[t, best]:
                    best = e
            idx[t, j] = best
            remaining.remove(best)
    return idx


def _brute_ffn(x, w13, w2, act):
    f = w2.shape[1]
    if act == "swiglu":
        g = np.einsum("td,fd->tf", x, w13[:f])
        u = np.einsum("td,fd->tf", x, w13[f:])
        h = g * sps.expit(g) * u
    else:
        a = np.einsum("td,fd->tf", x, w13)
        h = a * sst.norm.cdf(a)
    return np.einsum("tf,df->td", h, w2)


def brute_layer(x, w_r, w13, w2, k, score, act, cap, logit_bias=None, sel_bias=None,
                sw13=None, sw2=None):
    T = x.shape[0]
    E = w13.shape[0]
    logits = np.einsum("td,ed->te", x, w_r)
    if logit_bias is not None:
        logits = logits + logit_bias
    scores = sps.softmax(logits, axis=1) if score == "softmax" else sps.expit(logits)
    key = scores + (sel_bias if sel_bias is not None else 0.0)
    idx = _brute_select(key, k)
    sel = np.zeros((T, E), dtype=bool)
    np.put_along_axis(sel, idx, True, axis=1)
    gate = np.zeros((T, E))
    for t in range(T):
        ch = idx[t]
        if score == "softmax":   # renormalised softmax top-k == softmax over chosen logits
            gate[t, ch] = np.exp(logits[t, ch] - sps.logsumexp(logits[t, ch]))
        else:
            gate[t, ch] = scores[t, ch] / scores[t, ch].sum()
    earlier = np.cumsum(sel, axis=0) - sel          # tokens before t routed to e
    kept = sel if cap is None else sel & (earlier < cap)
    Y = np.zeros_like(x)
    for e in range(E):
        Y += (kept[:, e] * gate[:, e])[:, None] * _brute_ffn(x, w13[e], w2[e], act)
    if sw13 is not None:
        for s in range(sw13.shape[0]):
            Y += _brute_ffn(x, sw13[s], sw2[s], act)
    return dict(Y=Y, idx=idx, kept=kept, scores=scores)


VARIANTS = [
    dict(score="softmax", act="swiglu", cf=None),
    dict(score="softmax", act="gelu", cf=None),
    dict(score="softmax", act="swiglu", cf=0.75),
    dict(score="softmax", act="gelu", cf=1.0, logit_bias={0: 2.0, 3: 2.0}),
    dict(score="sigmoid", act="swiglu", cf=None, sel_bias=True, n_shared=1),
    dict(score="softmax", act="swiglu", cf=1.25, n_shared=1),
]


@pytest.mark.parametrize("var", VARIANTS)
def test_sparse_oracle_equals_dense_brute_force(var):
    w, g = _tiny(T=40, d=16, E=6, k=2, f=12, **var)
    cap = O.capacity(w.T, w.k, w.E, w.cf)
    fwd = O.layer_forward(g["x"], g["w_r"], g["w13"], g["w2"], w.k, w.score, w.act, cap,
                          g["logit_bias"], g["sel_bias"], g["sw13"], g["sw2"])
    bf = brute_layer(g["x"], g["w_r"], g["w13"], g["w2"], w.k, w.score, w.act, cap,
                     g["logit_bias"], g["sel_bias"], g["sw13"], g["sw2"])
    np.testing.assert_array_equal(fwd["router"]["topk_idx"], bf["idx"])
    np.testing.assert_allclose(fwd["router"]["scores"], bf["scores"], rtol=1e-13, atol=1e-15)
    kept_o = np.zeros_like(bf["kept"])
    for t in range(w.T):
        for j in range(w.k):
            if fwd["perm"]["row_of"][t, j] >= 0:
                kept_o[t, fwd["router"]["topk_idx"][t, j]] = True
    np.testing.assert_array_equal(kept_o, bf["kept"])
    np.testing.assert_allclose(fwd["Y"], bf["Y"], rtol=1e-11, atol=1e-12)


def test_tiny_fp32_workload_full_size_brute_force():
    """The whole tiny fp32 workload (T=256, d=128, E=8, k=2, f=256)."""
    from moe_inputs import WORKLOADS
    w = WORKLOADS["tiny_fp32"]
    g = {n: as_f64(v, w.dtype) for n, v in gen_all(w).items()}
    fwd = O.layer_forward(g["x"], g["w_r"], g["w13"], g["w2"], w.k, w.score, w.act, None)
    bf = brute_layer(g["x"], g["w_r"], g["w13"], g["w2"], w.k, w.score, w.act, None)
    np.testing.assert_array_equal(fwd["router"]["topk_idx"], bf["idx"])
    np.testing.assert_allclose(fwd["Y"], bf["Y"], rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------- closed forms
def test_zero_router_weight_tie_break_and_stats():
    w, g = _tiny(T=10, E=5, k=3)
    r = O.router_forward(g["x"], np.zeros_like(g["w_r"]), w.k)
    assert (r["topk_idx"] == np.arange(3)[None, :]).all()
    np.testing.assert_allclose(r["gates"], 1.0 / 3.0, rtol=0, atol=1e-15)
    st = O.aux_stats(r["scores"], r["topk_idx"], w.E)
    np.testing.assert_allclose(st["z"], 1.0 / w.E, rtol=1e-15)
    np.testing.assert_allclose(st["y"], [1 / 3, 1 / 3, 1 / 3, 0, 0], rtol=1e-15)
    assert abs(st["S"] - 1.0 / w.E) < 1e-15 and abs(st["L_aux"] - 1.0) < 1e-14


def test_k_equals_E_gives_full_softmax():
    w, g = _tiny(T=12, E=5, k=5)
    r = O.router_forward(g["x"], g["w_r"], 5)
    full = sps.softmax(g["x"] @ g["w_r"].T, axis=1)
    np.testing.assert_allclose(np.take_along_axis(full, r["topk_idx"], 1), r["gates"], rtol=1e-13)
    assert (np.diff(np.take_along_axis(full, r["topk_idx"], 1), axis=1) <= 0).all()


def test_uniform_counts_give_unit_aux_loss():
    T, E, k = 64, 8, 2
    idx = np.stack([(np.arange(T) * k + j) % E for j in range(k)], axis=1)
    rng = np.random.default_rng(3)
    scores = sps.softmax(rng.standard_normal((T, E)), axis=1)
    st = O.aux_stats(scores, idx, E)
    np.testing.assert_array_equal(st["counts"], np.full(E, T * k // E))
    assert abs(st["L_aux"] - 1.0) < 1e-14


def test_golden_uniform_top2_ratio():
    (T, k, E, want), = _read_golden("uniform_top2_ratio.txt")
    T, k, E, want = int(T), int(k), int(E), float(want)
    idx = np.stack([(np.arange(T) * k + j) % E for j in range(k)], axis=1)
    st = O.aux_stats(np.full((T, E), 1.0 / E), idx, E)
    assert abs(np.sort(st["y"])[-2:].sum() - want) < 1e-15
    assert abs(st["y"].sum() - 1.0) < 1e-15


def test_hand_computed_aux_stats():
    # T=4, E=2, k=1: tokens 0,1,2 -> expert 0, token 3 -> expert 1
    scores = np.array([[0.9, 0.1], [0.6, 0.4], [0.7, 0.3], [0.2, 0.8]])
    idx = np.array([[0], [0], [0], [1]])
    st = O.aux_stats(scores, idx, 2)
    assert list(st["counts"]) == [3, 1]
    np.testing.assert_allclose(st["y"], [0.75, 0.25])
    np.testing.assert_allclose(st["z"], [0.6, 0.4])
    assert abs(st["S"] - (0.75 * 0.6 + 0.25 * 0.4)) < 1e-15
    assert abs(st["L_aux"] - 2 * 0.55) < 1e-15


def test_golden_capacity_worked_example():
    (T, k, E, cf, ideal, capv), = _read_golden("capacity_worked_example.txt")
    T, k, E, cf, ideal, capv = int(T), int(k), int(E), float(cf), int(ideal), int(capv)
    assert T * k // E == ideal
    assert O.capacity(T, k, E, cf) == capv
    assert O.capacity(T, k, E, None) is None


def test_capacity_rounds_up_a_fractional_limit():
    """The worked example's limit is an integer; where cf T k / E is not,
    the reading taken rounds up (a limit of 2.5 tokens keeps 3), so the
    limit is never below cf times the mean load."""
    assert O.capacity(10, 1, 4, 1.0) == 3            # 2.5
    assert O.capacity(3, 2, 4, 1.25) == 2            # 1.875
    assert O.capacity(8, 2, 8, 1.0) == 2             # exactly 2: no rounding
    assert O.capacity(7, 1, 3, 0.0) == 0


def test_capacity_keeps_first_tokens_when_all_go_to_one_expert():
    T, E, k, cap = 50, 4, 1, 7
    idx = np.full((T, k), 2)
    p = O.permute(idx, E, cap)
    assert list(p["offsets"]) == [0, 0, 0, cap, cap]
    assert list(p["token_of"]) == list(range(cap))
    assert (p["row_of"][:cap, 0] == np.arange(cap)).all() and (p["row_of"][cap:] == -1).all()
    assert p["n_dropped"] == T - cap


def test_capacity_zero_drops_everything():
    idx = np.array([[0, 1], [1, 2], [2, 0]])
    p = O.permute(idx, 3, 0)
    assert (p["row_of"] == -1).all() and p["n_dropped"] == 6 and p["offsets"][-1] == 0


def _torch_ffn(x, w13, w2, act):
    xt, a, b = torch.from_numpy(x), torch.from_numpy(w13), torch.from_numpy(w2)
    f = w2.shape[1]
    if act == "swiglu":
        h = torch.nn.functional.silu(xt @ a[:f].T) * (xt @ a[f:].T)
    else:
        h = torch.nn.functional.gelu(xt @ a.T, approximate="none")
    return (h @ b.T).numpy()


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_single_expert_is_textbook_ffn(act):
    w, g = _tiny(T=9, E=1, k=1, act=act)
    fwd = O.layer_forward(g["x"], g["w_r"], g["w13"], g["w2"], 1, act=act)
    np.testing.assert_allclose(fwd["Y"], _torch_ffn(g["x"], g["w13"][0], g["w2"][0], act),
                               rtol=1e-12, atol=1e-13)


def test_identical_experts_give_plain_ffn():
    w, g = _tiny(T=20, E=5, k=3)
    w13 = np.repeat(g["w13"][:1], 5, axis=0)
    w2 = np.repeat(g["w2"][:1], 5, axis=0)
    fwd = O.layer_forward(g["x"], g["w_r"], w13, w2, 3)
    np.testing.assert_allclose(fwd["Y"], _torch_ffn(g["x"], w13[0], w2[0], "swiglu"),
                               rtol=1e-12, atol=1e-13)


def test_shared_expert_alone_when_everything_drops():
    w, g = _tiny(T=16, E=4, k=2, n_shared=1)
    fwd = O.layer_forward(g["x"], g["w_r"], g["w13"], g["w2"], 2, cap=0, sw13=g["sw13"],
                          sw2=g["sw2"])
    np.testing.assert_allclose(fwd["Y"], _torch_ffn(g["x"], g["sw13"][0], g["sw2"][0], "swiglu"),
                               rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------- invariants
@pytest.mark.parametrize("cf", [None, 0.5, 1.0])
def test_routing_and_permutation_invariants(cf):
    w, g = _tiny(T=64, E=8, k=3, cf=cf)
    cap = O.capacity(w.T, w.k, w.E, cf)
    r = O.router_forward(g["x"], g["w_r"], w.k)
    np.testing.assert_allclose(r["gates"].sum(1), 1.0, rtol=0, atol=1e-14)
    for t in range(w.T):
        assert len(set(r["topk_idx"][t])) == w.k
    st = O.aux_stats(r["scores"], r["topk_idx"], w.E)
    assert st["counts"].sum() == w.T * w.k
    p = O.permute(r["topk_idx"], w.E, cap)
    A = p["offsets"][-1]
    assert (np.diff(p["offsets"]) >= 0).all() and A == w.T * w.k - p["n_dropped"]
    kept = p["row_of"][p["row_of"] >= 0]
    assert sorted(kept.tolist()) == list(range(A))
    for t in range(w.T):
        for j in range(w.k):
            rr = p["row_of"][t, j]
            if rr >= 0:
                assert p["token_of"][rr] == t
                e = r["topk_idx"][t, j]
                assert p["offsets"][e] <= rr < p["offsets"][e + 1]
    for e in range(w.E):
        seg = p["token_of"][p["offsets"][e]:p["offsets"][e + 1]]
        assert (np.diff(seg) > 0).all()
        if cap is not None:
            assert len(seg) == min(cap, st["counts"][e])


@pytest.mark.parametrize("k", [1, 3])
def test_unpermute_of_permute_is_k_times_identity(k):
    w, g = _tiny(T=30, E=6, k=k)
    r = O.router_forward(g["x"], g["w_r"], k)
    p = O.permute(r["topk_idx"], w.E)
    x_perm = g["x"][p["token_of"]]
    np.testing.assert_array_equal(O.permute_backward(x_perm, p["row_of"]), k * g["x"])


# --------------------------------------------------------- finite differences
def test_activation_derivatives():
    a = np.linspace(-6, 6, 101)
    h = 1e-6
    np.testing.assert_allclose(O.dsilu(a), (O.silu(a + h) - O.silu(a - h)) / (2 * h), atol=1e-8)
    np.testing.assert_allclose(O.dgelu(a), (O.gelu(a + h) - O.gelu(a - h)) / (2 * h), atol=1e-8)
    np.testing.assert_allclose(O.gelu(a), a * sst.norm.cdf(a), rtol=1e-13, atol=1e-15)


FD_VARIANTS = [
    dict(score="softmax", act="swiglu", cf=None, aux_coef=0.0),
    dict(score="softmax", act="swiglu", cf=0.75, aux_coef=0.3),
    dict(score="softmax", act="gelu", cf=None, aux_coef=0.0, logit_bias={1: 0.5}),
    dict(score="sigmoid", act="swiglu", cf=None, aux_coef=0.2, sel_bias=True, n_shared=1),
]


@pytest.mark.parametrize("var", FD_VARIANTS)
def test_gradients_by_central_differences(var):
    var = dict(var)   # the parametrized dict is shared with other tests
    aux = var.pop("aux_coef")
    # seed chosen so no token sits within 1e-3 of a top-k boundary
    for seed in range(50):
        w, g = _tiny(T=10, d=6, E=5, k=2, f=4, seed=seed, **var)
        # scale the router up so its gradient is not tiny next to the FFN's
        g["w_r"] = g["w_r"] * 40.0
        r = O.router_forward(g["x"], g["w_r"], w.k, w.score, g["logit_bias"], g["sel_bias"])
        if not O.near_tie_tokens(r["key"], w.k, 1e-3).any():
            break
    else:
        pytest.fail("no tie-free seed")
    cap = O.capacity(w.T, w.k, w.E, w.cf)
    params = dict(x=g["x"], w_r=g["w_r"], w13=g["w13"], w2=g["w2"])
    if w.n_shared:
        params.update(sw13=g["sw13"], sw2=g["sw2"])
    dY = g["dy"]

    def loss(p):
        f = O.layer_forward(p["x"], p["w_r"], p["w13"], p["w2"], w.k, w.score, w.act, cap,
                            g["logit_bias"], g["sel_bias"], p.get("sw13"), p.get("sw2"))
        return float((f["Y"] * dY).sum()) + aux * f["stats"]["L_aux"], f

    _, fwd = loss(params)
    bwd = O.layer_backward(fwd, params["x"], params["w_r"], params["w13"], params["w2"], dY,
                           w.score, w.act, aux, params.get("sw13"), params.get("sw2"))
    analytic = dict(x=bwd["dX"], w_r=bwd["dw_r"], w13=bwd["dw13"], w2=bwd["dw2"],
                    sw13=bwd["dsw13"], sw2=bwd["dsw2"])
    h = 1e-6
    for name, val in params.items():
        num = np.zeros_like(val)
        for i in np.ndindex(val.shape):
            p2 = {n: v.copy() for n, v in params.items()}
            p2[name][i] += h
            lp, _ = loss(p2)
            p2[name][i] -= 2 * h
            lm, _ = loss(p2)
            num[i] = (lp - lm) / (2 * h)
        scale = max(1.0, np.abs(num).max())
        np.testing.assert_allclose(analytic[name], num, rtol=0, atol=2e-6 * scale,
                                   err_msg=name)


def test_aux_gradient_is_not_dropped():
    """The aux term must change dW_r (a dropped aux term fails this)."""
    w, g = _tiny(T=12, d=6, E=4, k=2, f=4)
    fwd = O.layer_forward(g["x"], g["w_r"], g["w13"], g["w2"], 2)
    b0 = O.layer_backward(fwd, g["x"], g["w_r"], g["w13"], g["w2"], g["dy"], aux_coef=0.0)
    b1 = O.layer_backward(fwd, g["x"], g["w_r"], g["w13"], g["w2"], g["dy"], aux_coef=1.0)
    assert np.abs(b1["dw_r"] - b0["dw_r"]).max() > 1e-6


# ------------------------------------------------------------- near ties
def test_near_tie_flags():
    key = np.array([[0.5, 0.3, 0.2 + 5e-6, 0.2, 0.0],
                    [0.5, 0.3, 0.1, 0.05, 0.05],
                    [0.4, 0.4 - 1e-7, 0.1, 0.05, 0.05]])
    flags = O.near_tie_tokens(key, 2)
    assert list(flags) == [False, False, True]
    assert list(O.near_tie_tokens(key, 3)) == [True, False, True]


# ---------------------------------------------------------------- generator
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(100000) * 3).astype(np.float32)
    v[:4] = [1.00390625, 1.01171875, -1.00390625, 0.0]   # exact ties
    ours = to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ours),
                                  torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_per_expert():
    from moe_inputs import gen_expert_w13, gen_w13
    w = Workload("g", T=8, d=16, E=4, k=2, f=8)
    a = gen_w13(w)
    np.testing.assert_array_equal(a[2], gen_expert_w13(w, 2))
    np.testing.assert_array_equal(a, gen_w13(w, threads=1))
    assert not np.array_equal(a[0], a[1])


# -------------------------------------------- bias update and z-loss pins
def test_bias_update_rule():
    # T k = 12 assignments over E = 4 experts: target 3 each
    b = np.array([0.5, 0.0, -0.25, 0.1])
    counts = np.array([5, 3, 1, 3])
    nb = O.bias_update(b, counts, T=6, k=2, gamma=1e-3)
    np.testing.assert_allclose(nb, [0.5 - 1e-3, 0.0, -0.25 + 1e-3, 0.1], rtol=0, atol=1e-15)
    # uniform load leaves the bias unchanged
    assert (O.bias_update(b, np.full(4, 3), 6, 2, 1e-3) == b).all()


def test_bias_update_balances_a_skewed_router():
    """Repeated updates move the selection toward balance ([Recipe] §5.3)."""
    rng = np.random.default_rng(5)
    T, E, k = 400, 8, 2
    logits = rng.standard_normal((T, E)) * 0.3
    logits[:, 0] += 1.5
    scores = sps.softmax(logits, axis=1)
    b = np.zeros(E)
    spread = []
    for _ in range(300):
        idx = np.argsort(-(scores + b), axis=1, kind="stable")[:, :k]
        counts = np.bincount(idx.ravel(), minlength=E)
        spread.append(counts.max() - counts.min())
        b = O.bias_update(b, counts, T, k, 2e-3)
    assert spread[-1] < spread[0] / 3


def test_z_loss_closed_form_and_gradient():
    T, E = 5, 6
    assert abs(O.z_loss(np.zeros((T, E))) - np.log(E) ** 2) < 1e-14
    rng = np.random.default_rng(2)
    l = rng.standard_normal((T, E)) * 2
    g = O.z_loss_grad(l)
    h = 1e-6
    num = np.zeros_like(l)
    for i in np.ndindex(l.shape):
        lp = l.copy(); lp[i] += h
        lm = l.copy(); lm[i] -= h
        num[i] = (O.z_loss(lp) - O.z_loss(lm)) / (2 * h)
    np.testing.assert_allclose(g, num, rtol=0, atol=1e-8)
    # shifting every logit of a token by c shifts its lse by c
    np.testing.assert_allclose(O.router_logsumexp(l + 3.0), O.router_logsumexp(l) + 3.0, rtol=1e-14)


def test_layer_gradient_with_z_loss_by_central_differences():
    for seed in range(50):
        w, g = _tiny(T=8, d=6, E=5, k=2, f=4, seed=seed)
        g["w_r"] = g["w_r"] * 40.0
        r = O.router_forward(g["x"], g["w_r"], w.k)
        if not O.near_tie_tokens(r["key"], w.k, 1e-3).any():
            break
    zc = 0.5

    def loss(x, w_r):
        f = O.layer_forward(x, w_r, g["w13"], g["w2"], w.k)
        return float((f["Y"] * g["dy"]).sum()) + zc * O.z_loss(f["router"]["logits"]), f

    _, fwd = loss(g["x"], g["w_r"])
    bwd = O.layer_backward(fwd, g["x"], g["w_r"], g["w13"], g["w2"], g["dy"], z_coef=zc)
    h = 1e-6
    for name, val, ana in (("x", g["x"], bwd["dX"]), ("w_r", g["w_r"], bwd["dw_r"])):
        num = np.zeros_like(val)
        for i in np.ndindex(val.shape):
            v2 = val.copy(); v2[i] += h
            lp, _ = loss(v2, g["w_r"]) if name == "x" else loss(g["x"], v2)
            v2[i] -= 2 * h
            lm, _ = loss(v2, g["w_r"]) if name == "x" else loss(g["x"], v2)
            num[i] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(ana, num, rtol=0, atol=2e-6 * max(1.0, np.abs(num).max()),
                                   err_msg=name)


# ------------------------------------------------------------ noisy gate
def test_gumbel_noise_hand_values():
    """u = exp(-exp(-c)) gives Gumbel noise c (up to the eps of [Balance])."""
    c = np.array([-1.5, 0.0, 0.7, 2.0])
    u = np.exp(-np.exp(-c))
    np.testing.assert_allclose(O.gumbel_noise(u), c, rtol=0, atol=1e-8)
    # u -> 0 and u -> 1 stay finite thanks to eps
    assert np.isfinite(O.gumbel_noise(np.array([0.0, 1.0 - 2**-24]))).all()


def test_gumbel_max_samples_the_softmax():
    """Gumbel-max: argmax(l + g) with g from uniform draws is distributed as
    softmax(l) (a property of the Gumbel law, checked statistically)."""
    rng = np.random.default_rng(11)
    l = np.array([0.3, -1.0, 1.2, 0.0, -0.4])
    n = 200_000
    u = rng.random((n, l.size))
    pick = np.argmax(l[None, :] + O.gumbel_noise(u), axis=1)
    freq = np.bincount(pick, minlength=l.size) / n
    p = np.exp(l) / np.exp(l).sum()
    assert (np.abs(freq - p) < 5 * np.sqrt(p * (1 - p) / n)).all(), (freq, p)


def test_noisy_router_worked_example_and_top1():
    """One token, three experts, noise c = (0, 1, -1), tau = 0.5: scores are
    softmax((l + c) / tau) by hand; with k = 1 the choice is argmax(l + c)."""
    x = np.array([[1.0, 0.0]])
    w_r = np.array([[0.2, 0.0], [-0.3, 0.0], [0.9, 0.0]])
    c = np.array([0.0, 1.0, -1.0])
    u = np.exp(-np.exp(-c))[None, :]
    r = O.router_forward(x, w_r, 1, gumbel_u=u, tau=0.5)
    z = (np.array([0.2, -0.3, 0.9]) + c) / 0.5
    want = np.exp(z) / np.exp(z).sum()
    np.testing.assert_allclose(r["scores"][0], want, rtol=1e-8)
    assert r["topk_idx"][0, 0] == int(np.argmax(np.array([0.2, -0.3, 0.9]) + c)) == 1
    assert r["gates"][0, 0] == 1.0
    with pytest.raises(ValueError):
        O.router_forward(x, w_r, 1, score="sigmoid", gumbel_u=u, tau=0.5)


def test_layer_gradient_with_noisy_gate_by_central_differences():
    """Fixed draws make the noisy layer deterministic: its dX and dW_r
    (including the aux and z-loss terms and the 1/tau chain factor) match
    central differences."""
    for seed in range(50):
        w, g = _tiny(T=8, d=6, E=5, k=2, f=4, seed=seed, gumbel_tau=0.7)
        g["w_r"] = g["w_r"] * 40.0
        r = O.router_forward(g["x"], g["w_r"], w.k, gumbel_u=g["gumbel_u"], tau=0.7)
        if not O.near_tie_tokens(r["key"], w.k, 1e-3).any():
            break
    ac, zc, tau = 0.3, 0.2, 0.7

    def loss(x, w_r):
        f = O.layer_forward(x, w_r, g["w13"], g["w2"], w.k, gumbel_u=g["gumbel_u"], tau=tau)
        st = f["stats"]
        # the aux gradient holds y fixed: differentiate E * sum_i y_i z_i with y frozen
        aux = w.E * float((y_fixed * st["z"]).sum())
        return (float((f["Y"] * g["dy"]).sum()) + ac * aux
                + zc * O.z_loss(f["router"]["logits"])), f

    y_fixed = O.layer_forward(g["x"], g["w_r"], g["w13"], g["w2"], w.k, gumbel_u=g["gumbel_u"],
                              tau=tau)["stats"]["y"]
    _, fwd = loss(g["x"], g["w_r"])
    bwd = O.layer_backward(fwd, g["x"], g["w_r"], g["w13"], g["w2"], g["dy"], aux_coef=ac,
                           z_coef=zc, tau=tau)
    h = 1e-6
    for name, val, ana in (("x", g["x"], bwd["dX"]), ("w_r", g["w_r"], bwd["dw_r"])):
        num = np.zeros_like(val)
        for i in np.ndindex(val.shape):
            v2 = val.copy(); v2[i] += h
            lp, _ = loss(v2, g["w_r"]) if name == "x" else loss(g["x"], v2)
            v2[i] -= 2 * h
            lm, _ = loss(v2, g["w_r"]) if name == "x" else loss(g["x"], v2)
            num[i] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(ana, num, rtol=1e-5, atol=1e-7, err_msg=name)


def test_router_backward_on_a_token_subset():
    """Rows of the router gradient are independent given the batch's y and T:
    evaluating a subset with n_tokens = T reproduces those rows of the full
    batch (aux and z-loss terms included)."""
    w, g = _tiny(T=40, d=8, E=6, k=2, f=4, seed=3)
    r = O.router_forward(g["x"], g["w_r"], w.k)
    st = O.aux_stats(r["scores"], r["topk_idx"], w.E)
    dgate = np.random.default_rng(4).standard_normal((w.T, w.k))
    full = O.router_backward(g["x"], g["w_r"], r["scores"], r["topk_idx"], r["gates"], dgate,
                             aux_coef=0.3, y=st["y"], z_coef=0.2, logits=r["logits"])
    sub = np.array([1, 7, 22, 39])
    part = O.router_backward(g["x"][sub], g["w_r"], r["scores"][sub], r["topk_idx"][sub],
                             r["gates"][sub], dgate[sub], aux_coef=0.3, y=st["y"], z_coef=0.2,
                             logits=r["logits"][sub], n_tokens=w.T)
    np.testing.assert_allclose(part["dlogits"], full["dlogits"][sub], rtol=1e-13, atol=1e-15)


def test_row_comparison_ignores_slot_order_only():
    """The GPU-vs-oracle row comparison keys rows by (token, expert): a
    swapped slot order with the same rows passes, a wrong row does not."""
    import pytest
    from parity_util import assert_rows_match
    o_idx = np.array([[3, 1], [0, 2]])
    o_row = np.array([[5, 1], [0, 3]])
    g_idx = np.array([[1, 3], [0, 2]])
    assert_rows_match(g_idx, np.array([[1, 5], [0, 3]]), o_idx, o_row)
    with pytest.raises(AssertionError):
        assert_rows_match(g_idx, np.array([[5, 1], [0, 3]]), o_idx, o_row)
    with pytest.raises(AssertionError):
        assert_rows_match(np.array([[1, 4], [0, 2]]), np.array([[1, 5], [0, 3]]), o_idx, o_row)


# ------------------------------------------------------------------ FP8 forward
def _torch_e4m3_codes(v):
    import torch
    return torch.from_numpy(np.asarray(v, dtype=np.float64)).to(torch.float32) \
        .to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_matches_library_on_every_code():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    assert (np.isnan(ref) == np.isnan(got)).all()
    fin = ~np.isnan(ref)
    assert (ref[fin] == got[fin]).all()
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9 and got[0x7F] != got[0x7F]


def test_e4m3_encode_matches_library_rounding():
    """Every finite bf16 value within +-448, random fp32 values, and exact
    ties, against torch's float32 -> float8_e4m3fn cast (round to nearest even)."""
    u = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    u = u[np.isfinite(u)].astype(np.float64)
    u = u[np.abs(u) <= 448]
    rng = np.random.default_rng(5)
    r = (rng.standard_normal(20000) * np.exp2(rng.integers(-12, 8, 20000))).astype(np.float32)
    r = r[np.abs(r) <= 448].astype(np.float64)
    for v in (u, r):
        assert (O.e4m3_encode(v) == _torch_e4m3_codes(v)).all()
    # hand ties: halfway values go to the even mantissa
    assert O.e4m3_encode([1.0625, 1.1875, 3 * 2.0 ** -10, 2.0 ** -10, 240.0])[:].tolist() == \
        [0x38, 0x3A, 0x02, 0x00, 0x77]
    assert O.e4m3_encode([-2.0 ** -11])[0] == 0x80      # sign kept on rounding to zero


def test_fp8_row_scale_is_the_smallest_power_of_two():
    amax = np.array([448.0, 449.0, 224.0, 224.5, 1.0, 1.75, 1.76, 0.0, 3e-5, 6e4])
    got = O.fp8_row_scale_exp(amax)
    for a, e in zip(amax, got):
        if a == 0:
            assert e == 0
            continue
        want = next(x for x in range(-60, 60) if a <= 448.0 * 2.0 ** x)   # brute force
        assert e == want, (a, e, want)


def test_quantize_rows_error_and_range():
    rng = np.random.default_rng(6)
    X = rng.standard_normal((40, 96)) * np.exp2(rng.integers(-20, 20, 40))[:, None]
    X = O.round_bf16(X)
    q, e = O.quantize_rows_fp8(X)
    D = O.dequantize_rows_fp8(q, e)
    scaled = np.abs(D) * np.exp2(-e.astype(float))[:, None]
    assert (scaled.max(axis=1) <= 448).all() and (scaled.max(axis=1) > 224 * 0.9).all()
    s = np.exp2(e.astype(float))[:, None]
    normal = np.abs(X) >= 2.0 ** -6 * s
    err = np.abs(D - X)
    assert (err[normal] <= 2.0 ** -4 * np.abs(X[normal]) * (1 + 1e-12)).all()
    assert (err[~normal] <= (2.0 ** -10 * s + 0 * X)[~normal]).all()


def test_round_bf16_matches_library():
    import torch
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(50000) * np.exp2(rng.integers(-30, 30, 50000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert (O.round_bf16(v.astype(np.float64)) == ref).all()


def _brute_fp8_rows(M):
    """Dequantized per-row FP8 by brute force: scale exponent by search, codes
    by torch's own cast."""
    out = np.zeros_like(M)
    for i, row in enumerate(M):
        a = np.abs(row).max()
        e = 0 if a == 0 else next(x for x in range(-60, 60) if a <= 448.0 * 2.0 ** x)
        codes = _torch_e4m3_codes(row / 2.0 ** e)
        out[i] = O.e4m3_decode(codes) * 2.0 ** e
    return out


# ------------------------------------------------------------------ FP8 backward
@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_expert_backward_fp8_brute_force(act):
    """The FP8 expert backward against explicit loops: bf16 dO and W2^T
    quantized per row by brute force (scale search + library E4M3 cast), the
    activation backward written out on the bf16 pre-activations, bf16 dpre
    and W13^T quantized the same way; the weight gradients on the unquantized
    values."""
    rng = np.random.default_rng(18)
    n, d, f = 4, 32, 16
    P = 2 * f if act == "swiglu" else f
    X = O.round_bf16(rng.standard_normal((n, d)))
    w13 = O.round_bf16(rng.standard_normal((P, d)) / 5)
    w2 = O.round_bf16(rng.standard_normal((d, f)) / 4)
    _, saved = O.expert_forward(X, w13, w2, act)
    dO = rng.standard_normal((n, d)) * 0.3
    dOd = _brute_fp8_rows(O.round_bf16(dO))
    W2t = _brute_fp8_rows(w2.T.copy())          # [f, d]
    W13t = _brute_fp8_rows(w13.T.copy())        # [d, P]
    dH = np.array([[sum(dOd[t, c] * W2t[j, c] for c in range(d)) for j in range(f)]
                   for t in range(n)])
    a = O.round_bf16(saved["a"])                 # the stored bf16 pre-activations
    sg = 1 / (1 + np.exp(-a))
    if act == "swiglu":
        b = O.round_bf16(saved["b"])
        dpre = np.concatenate([dH * b * sg * (1 + a * (1 - sg)), dH * a * sg], axis=1)
    else:
        cdf = 0.5 * (1 + sps.erf(a / np.sqrt(2)))
        dpre = dH * (cdf + a * np.exp(-a * a / 2) / np.sqrt(2 * np.pi))
    dpd = _brute_fp8_rows(O.round_bf16(dpre))
    dX = np.array([[sum(dpd[t, p] * W13t[j, p] for p in range(P)) for j in range(d)]
                   for t in range(n)])
    gX, g13, g2, gpre = O.expert_backward_fp8_wq(X, O.quantize_weights_fp8_t(w2),
                                                 O.quantize_weights_fp8_t(w13), saved, dO, act)
    np.testing.assert_allclose(gpre, dpre, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gX, dX, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g2, dO.T @ saved["H"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g13, dpre.T @ X, rtol=1e-12, atol=1e-14)
    # and it stays near the exact backward (quantization error only)
    ex, _, _, _ = O.expert_backward(X, w13, w2, saved, dO, act)
    assert np.abs(gX - ex).max() < 0.15 * np.abs(ex).max()


def test_expert_backward_fp8_exact_with_per_channel_scales():
    """When every quantized value is representable, the FP8 backward equals
    the exact backward bit for bit. Each weight here has one dominant input
    channel: scaled per input channel (rows of the transpose) every value
    stays exact, while scaling per output channel would push the small
    entries into E4M3's subnormal range and round them; the test checks that
    this wrong axis does change dX, so the pin can catch it."""
    n, d, f = 6, 16, 8
    P = 2 * f
    j0, c0 = 3, 5                                  # dominant input channels of w2, w13
    small = np.array([1.125, -0.5, 0.75, -1.125, 0.5, -0.75]) * 0.25
    w2 = np.resize(small, (d, f)).astype(np.float64)
    w2[:, j0] = 448.0 * 2 ** 6                     # input channel j0 of the down-projection
    w13 = np.resize(small[::-1], (P, d)).astype(np.float64)
    w13[:, c0] = -448.0 * 2 ** 5                   # input channel c0 of the up-projection
    X = np.resize(small, (n, d)) * 4
    # a = 0: silu = 0, silu' = 1/2; b = 1 except b[:, j0] = 0 (kills the big column of dH)
    a = np.zeros((n, f))
    b = np.ones((n, f))
    b[:, j0] = 0.0
    saved = dict(a=a, b=b, H=O.silu(a) * b)
    dO = np.zeros((n, d))
    for t in range(n):
        dO[t, (2 * t + 1) % d] = 1.0               # one-hot upstream rows
    exact = O.expert_backward(X, w13, w2, saved, dO, "swiglu")
    got = O.expert_backward_fp8_wq(X, O.quantize_weights_fp8_t(w2), O.quantize_weights_fp8_t(w13),
                                   saved, dO, "swiglu")
    for g, e in zip(got, exact):
        assert np.array_equal(g, e)
    # the wrong axis (one scale per output channel, i.e. per row of w) loses the small entries
    wrong = O.expert_backward_fp8_wq(X, O.quantize_weights_fp8(w2).T,
                                     O.quantize_weights_fp8(w13).T, saved, dO, "swiglu")
    assert not np.allclose(wrong[0], exact[0], rtol=1e-3, atol=0)


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_expert_forward_fp8_brute_force(act):
    """The FP8 expert forward against explicit loops over brute-force
    quantized operands (scale search + library E4M3 cast)."""
    rng = np.random.default_rng(8)
    n, d, f = 5, 64, 32
    X = O.round_bf16(rng.standard_normal((n, d)))
    P = 2 * f if act == "swiglu" else f
    w13 = O.round_bf16(rng.standard_normal((P, d)) / 8)
    w2 = O.round_bf16(rng.standard_normal((d, f)) / 6)
    Xd, Wd, W2d = _brute_fp8_rows(X), _brute_fp8_rows(w13), _brute_fp8_rows(w2)
    pre = np.array([[sum(Xd[t, c] * Wd[j, c] for c in range(d)) for j in range(P)]
                    for t in range(n)])
    if act == "swiglu":
        a, b = pre[:, :f], pre[:, f:]
        H = a / (1 + np.exp(-a)) * b
    else:
        H = O.gelu(pre)
    Hd = _brute_fp8_rows(O.round_bf16(H))
    Oref = np.array([[sum(Hd[t, c] * W2d[j, c] for c in range(f)) for j in range(d)]
                     for t in range(n)])
    got, sv = O.expert_forward_fp8(X, w13, w2, act)
    np.testing.assert_allclose(sv["a"], pre[:, :f] if act == "swiglu" else pre, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got, Oref, rtol=1e-12, atol=1e-12)
    # and it stays near the exact forward (quantization error only)
    exact, _ = O.expert_forward(X, w13, w2, act)
    assert np.abs(got - exact).max() < 0.15 * np.abs(exact).max()


# ------------------------------------------------------- FP8 block scales
def _brute_fp8_blocks(M, block=32):
    """Dequantized block-scaled FP8 by brute force: per block of `block`
    elements along a row, the exponent by search (clipped to [-127, 127]),
    codes by torch's own cast."""
    out = np.zeros_like(M)
    for i, row in enumerate(M):
        for j0 in range(0, row.size, block):
            blk = row[j0:j0 + block]
            a = np.abs(blk).max()
            e = 0 if a == 0 else next(x for x in range(-200, 200) if a <= 448.0 * 2.0 ** x)
            e = min(max(e, -127), 127)
            out[i, j0:j0 + block] = O.e4m3_decode(_torch_e4m3_codes(blk / 2.0 ** e)) * 2.0 ** e
    return out


def test_fp8_blocks_reduce_to_rows_for_one_block():
    """A row of at most one block quantizes exactly as the per-row scheme."""
    rng = np.random.default_rng(40)
    for K in (1, 16, 32):
        X = O.round_bf16(rng.standard_normal((20, K)) * np.exp2(rng.integers(-30, 30, 20))[:, None])
        qb, eb = O.quantize_blocks_fp8(X)
        qr, er = O.quantize_rows_fp8(X)
        assert (qb == qr).all() and (eb[:, 0] == er).all() and eb.shape == (20, 1)


def test_fp8_blocks_brute_force_and_partial_last_block():
    rng = np.random.default_rng(41)
    for K in (64, 96, 100, 208):
        X = O.round_bf16(rng.standard_normal((9, K)) * np.exp2(rng.integers(-12, 12, (9, 1))))
        X[:, :32] *= 1e3                          # blocks of different magnitude
        q, e = O.quantize_blocks_fp8(X)
        assert e.shape == (9, -(-K // 32))
        np.testing.assert_array_equal(O.dequantize_blocks_fp8(q, e), _brute_fp8_blocks(X))


def test_fp8_blocks_keep_small_blocks_that_a_row_scale_loses():
    """Each block takes its own scale: a block 2^20 below its row's largest
    block keeps E4M3 precision (error at most 2^-4 of each element), while one
    scale for the whole row rounds it to zero or subnormals."""
    rng = np.random.default_rng(42)
    big = 1.0 + rng.random(32)
    small = (1.0 + rng.random(32)) * 2.0 ** -20
    X = O.round_bf16(np.concatenate([big, small])[None, :])
    D = O.dequantize_blocks_fp8(*O.quantize_blocks_fp8(X))
    assert (np.abs(D - X) <= 2.0 ** -4 * np.abs(X) * (1 + 1e-12)).all()
    R = O.dequantize_rows_fp8(*O.quantize_rows_fp8(X))
    assert np.abs(R[0, 32:] - X[0, 32:]).max() > 0.5 * np.abs(X[0, 32:]).max()


def test_fp8_block_exponent_is_clipped_to_the_scale_range():
    X = np.zeros((3, 64))
    X[0, :32] = 2.0 ** -140                      # wants 2^-148: clipped to 2^-127
    X[1, 32:] = 1.0                              # block 0 all zero: exponent 0
    X[2, :] = 1.5 * 2.0 ** 100
    q, e = O.quantize_blocks_fp8(X)
    assert e.tolist() == [[-127, 0], [0, -8], [92, 92]]      # 1.5 * 2^100 <= 1.75 * 2^8 * 2^92
    assert (O.e4m3_decode(q[0, :32]) == 0).all()  # 2^-13 of the smallest subnormal step: zero


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_expert_forward_fp8_block_brute_force(act):
    """The block-scaled FP8 expert forward against explicit loops over
    operands quantized by brute force (scale search per block + library E4M3
    cast), with K = 40 and 24: a partial last block in both GEMMs."""
    rng = np.random.default_rng(43)
    n, d, f = 5, 40, 24
    P = 2 * f if act == "swiglu" else f
    X = O.round_bf16(rng.standard_normal((n, d)))
    X[:, 32:] *= 2.0 ** -9                       # the partial block far below the first
    w13 = O.round_bf16(rng.standard_normal((P, d)) / 6)
    w2 = O.round_bf16(rng.standard_normal((d, f)) / 5)
    Xd, W13d, W2d = _brute_fp8_blocks(X), _brute_fp8_blocks(w13), _brute_fp8_blocks(w2)
    pre = np.array([[sum(Xd[t, c] * W13d[j, c] for c in range(d)) for j in range(P)] for t in range(n)])
    if act == "swiglu":
        a, b = pre[:, :f], pre[:, f:]
        H = a / (1 + np.exp(-a)) * b
    else:
        H = 0.5 * pre * (1 + sps.erf(pre / np.sqrt(2)))
    Hd = _brute_fp8_blocks(O.round_bf16(H))
    out = np.array([[sum(Hd[t, j] * W2d[c, j] for j in range(f)) for c in range(d)] for t in range(n)])
    got, saved = O.expert_forward_fp8_block(X, w13, w2, act)
    np.testing.assert_allclose(got, out, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(saved["H"], H, rtol=1e-11, atol=1e-13)


# ------------------------------------------------ FP8 weight gradients
def test_expert_wgrad_fp8_brute_force():
    """FP8 weight gradients against explicit loops: every column of dO, H,
    dpre and X quantized by brute force over blocks of 32 tokens (40 tokens:
    one whole block and a partial one, with the partial block far smaller),
    after bf16 rounding of the values as stored (dpre here arrives in float64
    and must be rounded first)."""
    rng = np.random.default_rng(47)
    n, d, f = 40, 6, 5
    P = 2 * f
    X = O.round_bf16(rng.standard_normal((n, d)))
    H = O.round_bf16(rng.standard_normal((n, f)))
    dO = O.round_bf16(rng.standard_normal((n, d)))
    dpre = rng.standard_normal((n, P))                   # not bf16: the function rounds it
    for m in (X, H, dO, dpre):
        m[32:] *= 2.0 ** -9
    Xd, Hd, dOd = (_brute_fp8_blocks(m.T).T for m in (X, H, dO))
    dpd = _brute_fp8_blocks(O.round_bf16(dpre).T).T
    dw2 = np.array([[sum(dOd[t, c] * Hd[t, j] for t in range(n)) for j in range(f)] for c in range(d)])
    dw13 = np.array([[sum(dpd[t, r] * Xd[t, c] for t in range(n)) for c in range(d)] for r in range(P)])
    g13, g2 = O.expert_wgrad_fp8(X, H, dO, dpre)
    np.testing.assert_allclose(g2, dw2, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(g13, dw13, rtol=1e-12, atol=1e-15)


def test_fp8_wgrad_exact_on_block_exact_columns():
    """Columns whose 32-token blocks are E4M3 values times a power of two of
    their own (one element of each block in (224, 448] times it, so the
    block's scale is that power): the FP8 weight gradients equal the exact
    ones bit for bit. A scale per token row (the plausible mistake) cannot hold
    these columns, whose powers differ by up to 2^16 within a row."""
    rng = np.random.default_rng(48)
    codes = np.arange(256, dtype=np.uint8)
    vals = O.e4m3_decode(codes)
    mant = vals[(vals >= 1.0) & (vals <= 448.0)]
    top = mant[mant > 224.0]
    n, d, f = 72, 4, 3

    def block_exact(cols):
        m = rng.choice(mant, size=(n, cols))
        for b0 in range(0, n, 32):
            r = rng.integers(b0, min(b0 + 32, n), cols)
            m[r, np.arange(cols)] = rng.choice(top, cols)
            m[b0:b0 + 32] *= np.exp2(rng.integers(-8, 9, cols))
        return m * rng.choice([-1.0, 1.0], size=(n, cols))
    X, H, dO, dpre = block_exact(d), block_exact(f), block_exact(d), block_exact(2 * f)
    g13, g2 = O.expert_wgrad_fp8(X, H, dO, dpre)
    assert (g2 == dO.T @ H).all() and (g13 == dpre.T @ X).all()
    rows = O.dequantize_rows_fp8(*O.quantize_rows_fp8(dO))
    assert (rows != dO).any()


def test_grouped_backward_fp8_wgrad_is_per_expert():
    """With fp8_wgrad, each expert's weight gradients come from its own rows
    alone (token blocks restart at its first row): an expert of 40 tiny rows
    next to one of huge rows keeps the gradients of its own blocks, and the
    data gradients are untouched."""
    rng = np.random.default_rng(49)
    d, f, E = 8, 6, 2
    n0, n1 = 40, 24
    x_perm = O.round_bf16(rng.standard_normal((n0 + n1, d)))
    x_perm[:n0] *= 2.0 ** -20
    offsets = np.array([0, n0, n0 + n1])
    w13 = rng.standard_normal((E, 2 * f, d)) / 3
    w2 = rng.standard_normal((E, d, f)) / 3
    _, _, saved = O.grouped_ffn_forward(x_perm, offsets, w13, w2, "swiglu")
    dO = O.round_bf16(rng.standard_normal((n0 + n1, d)))
    ref = O.grouped_ffn_backward(x_perm, offsets, w13, w2, saved, dO, "swiglu")
    got = O.grouped_ffn_backward(x_perm, offsets, w13, w2, saved, dO, "swiglu", fp8_wgrad=True)
    np.testing.assert_array_equal(got["dx_perm"], ref["dx_perm"])
    for e, (lo, hi) in enumerate(((0, n0), (n0, n0 + n1))):
        g13, g2 = O.expert_wgrad_fp8(x_perm[lo:hi], saved["routed"][e]["H"], dO[lo:hi],
                                     ref["dpre"][lo:hi])
        np.testing.assert_array_equal(got["dw13"][e], g13)
        np.testing.assert_array_equal(got["dw2"][e], g2)
        # FP8 error of a sum over the expert's rows, relative to its own scale
        err = np.abs(got["dw13"][e] - ref["dw13"][e]).max() / np.abs(ref["dw13"][e]).max()
        assert err < 0.1, (e, err)


# ------------------------------------------------ E5M2 gradient operands
def _torch_e5m2_codes(v):
    import torch
    return torch.from_numpy(np.asarray(v, dtype=np.float64)).to(torch.float32) \
        .to(torch.float8_e5m2).view(torch.uint8).numpy()


def test_e5m2_decode_matches_library_on_every_code():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    got = O.e5m2_decode(codes)
    assert (np.isnan(ref) == np.isnan(got)).all() and (np.isinf(ref) == np.isinf(got)).all()
    fin = ~np.isnan(ref)
    assert (ref[fin] == got[fin]).all()
    assert np.nanmax(got[np.isfinite(got)]) == 57344.0 and got[1] == 2.0 ** -16


def test_e5m2_encode_matches_library_rounding():
    """Every finite bf16 value within +-57344, random fp32 values and hand ties,
    against torch's float32 -> float8_e5m2 cast (round to nearest even)."""
    u = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    u = u[np.isfinite(u)].astype(np.float64)
    u = u[np.abs(u) <= 57344]
    rng = np.random.default_rng(15)
    r = (rng.standard_normal(20000) * np.exp2(rng.integers(-20, 15, 20000))).astype(np.float32)
    r = r[np.abs(r) <= 57344].astype(np.float64)
    for v in (u, r):
        assert (O.e5m2_encode(v) == _torch_e5m2_codes(v)).all()
    # ties: 1.125 is halfway between 1.0 (mantissa 0) and 1.25 (mantissa 1) -> 1.0;
    # 1.375 between 1.25 and 1.5 -> 1.5 (even mantissa 2); 3 * 2^-17 -> 2 * 2^-16
    assert O.e5m2_encode([1.125, 1.375, 3 * 2.0 ** -17, 2.0 ** -17]).tolist() == [0x3C, 0x3E, 0x02, 0x00]
    assert O.e5m2_encode([-2.0 ** -18])[0] == 0x80


def test_e5m2_row_scale_is_the_smallest_power_of_two():
    amax = np.array([57344.0, 57345.0, 28672.0, 28673.0, 1.0, 1.75, 1.76, 0.0, 3e-5, 6e8])
    got = O.fp8_row_scale_exp(amax, "e5m2")
    for a, e in zip(amax, got):
        want = 0 if a == 0 else next(x for x in range(-80, 80) if a <= 57344.0 * 2.0 ** x)
        assert e == want, (a, e, want)


def _brute_fp8_rows_e5m2(M):
    """Dequantized per-row E5M2 by brute force: scale by search, codes by torch's cast."""
    out = np.zeros_like(M)
    for i, row in enumerate(M):
        a = np.abs(row).max()
        e = 0 if a == 0 else next(x for x in range(-80, 80) if a <= 57344.0 * 2.0 ** x)
        out[i] = O.e5m2_decode(_torch_e5m2_codes(row / 2.0 ** e)) * 2.0 ** e
    return out


def test_expert_backward_fp8_e5m2_gradients_brute_force():
    """The FP8 data gradients with E5M2 gradient operands (dO, dpre) against
    explicit loops over brute-force quantized operands: dO and dpre in E5M2,
    the transposed weights in E4M3."""
    rng = np.random.default_rng(19)
    n, d, f = 4, 32, 16
    P = 2 * f
    X = O.round_bf16(rng.standard_normal((n, d)))
    w13 = O.round_bf16(rng.standard_normal((P, d)) / 5)
    w2 = O.round_bf16(rng.standard_normal((d, f)) / 4)
    _, saved = O.expert_forward(X, w13, w2, "swiglu")
    dO = rng.standard_normal((n, d)) * 0.3
    dOd = _brute_fp8_rows_e5m2(O.round_bf16(dO))
    W2t, W13t = _brute_fp8_rows(w2.T.copy()), _brute_fp8_rows(w13.T.copy())
    dH = np.array([[sum(dOd[t, c] * W2t[j, c] for c in range(d)) for j in range(f)] for t in range(n)])
    a, b = O.round_bf16(saved["a"]), O.round_bf16(saved["b"])
    sg = 1 / (1 + np.exp(-a))
    dpre = np.concatenate([dH * b * sg * (1 + a * (1 - sg)), dH * a * sg], axis=1)
    dpd = _brute_fp8_rows_e5m2(O.round_bf16(dpre))
    dX = np.array([[sum(dpd[t, p] * W13t[j, p] for p in range(P)) for j in range(d)] for t in range(n)])
    gX, _, _, gpre = O.expert_backward_fp8_wq(X, O.quantize_weights_fp8_t(w2), O.quantize_weights_fp8_t(w13),
                                              saved, dO, "swiglu", grad_fmt="e5m2")
    np.testing.assert_allclose(gpre, dpre, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gX, dX, rtol=1e-12, atol=1e-14)
    # E5M2 keeps one mantissa bit less than E4M3: the two results differ
    gX4, _, _, _ = O.expert_backward_fp8_wq(X, O.quantize_weights_fp8_t(w2),
                                            O.quantize_weights_fp8_t(w13), saved, dO, "swiglu")
    assert (gX4 != gX).any()


def test_expert_wgrad_fp8_e5m2_gradients_brute_force():
    """FP8 weight gradients with E5M2 gradient columns (dO, dpre) and E4M3
    activation columns (H, X), blocks of 32 tokens, against explicit loops."""
    rng = np.random.default_rng(50)
    n, d, f = 40, 5, 4
    X = O.round_bf16(rng.standard_normal((n, d)))
    H = O.round_bf16(rng.standard_normal((n, f)))
    dO = O.round_bf16(rng.standard_normal((n, d)))
    dpre = rng.standard_normal((n, 2 * f))
    for m in (X, H, dO, dpre):
        m[32:] *= 2.0 ** -12

    def brute_cols(M, e5):
        out = np.zeros_like(M)
        for c in range(M.shape[1]):
            for b0 in range(0, M.shape[0], 32):
                blk = M[b0:b0 + 32, c]
                a = np.abs(blk).max()
                top = 57344.0 if e5 else 448.0
                e = 0 if a == 0 else next(x for x in range(-200, 200) if a <= top * 2.0 ** x)
                e = min(max(e, -127), 127)
                codes = (_torch_e5m2_codes if e5 else _torch_e4m3_codes)(blk / 2.0 ** e)
                out[b0:b0 + 32, c] = (O.e5m2_decode if e5 else O.e4m3_decode)(codes) * 2.0 ** e
        return out
    Xd, Hd = brute_cols(X, False), brute_cols(H, False)
    dOd, dpd = brute_cols(dO, True), brute_cols(O.round_bf16(dpre), True)
    g13, g2 = O.expert_wgrad_fp8(X, H, dO, dpre, grad_fmt="e5m2")
    np.testing.assert_allclose(g2, dOd.T @ Hd, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(g13, dpd.T @ Xd, rtol=1e-12, atol=1e-15)


# ------------------------------------------------ FP8 square-block weights
def _brute_fp8_squares(M, block=32):
    """Dequantized square-block FP8 by brute force: per block x block square
    (edges partial), the largest magnitude by explicit loops, the exponent by
    search (clipped to [-127, 127]), codes by torch's own E4M3 cast."""
    R, C = M.shape
    out = np.zeros_like(M)
    for i0 in range(0, R, block):
        for j0 in range(0, C, block):
            a = 0.0
            for i in range(i0, min(i0 + block, R)):
                for j in range(j0, min(j0 + block, C)):
                    a = max(a, abs(M[i, j]))
            e = 0 if a == 0 else next(x for x in range(-200, 200) if a <= 448.0 * 2.0 ** x)
            e = min(max(e, -127), 127)
            sq = M[i0:i0 + block, j0:j0 + block]
            out[i0:i0 + block, j0:j0 + block] = O.e4m3_decode(_torch_e4m3_codes(sq / 2.0 ** e)) * 2.0 ** e
    return out


def _brute_fp8_blocks_fmt(M, e5, block=32):
    """_brute_fp8_blocks in E4M3 or E5M2 (largest finite 448 or 57344)."""
    top = 57344.0 if e5 else 448.0
    out = np.zeros_like(M)
    for i, row in enumerate(M):
        for j0 in range(0, row.size, block):
            blk = row[j0:j0 + block]
            a = np.abs(blk).max()
            e = 0 if a == 0 else next(x for x in range(-200, 200) if a <= top * 2.0 ** x)
            e = min(max(e, -127), 127)
            codes = (_torch_e5m2_codes if e5 else _torch_e4m3_codes)(blk / 2.0 ** e)
            out[i, j0:j0 + block] = (O.e5m2_decode if e5 else O.e4m3_decode)(codes) * 2.0 ** e
    return out


def test_fp8_squares_brute_force_with_partial_edges():
    """Squares of very different magnitude, whole and partial at the bottom
    and right edges, against the brute force; the exponent array has one
    entry per square."""
    rng = np.random.default_rng(60)
    for R, C in ((32, 32), (70, 45), (33, 64), (96, 100)):
        W = rng.standard_normal((R, C))
        W *= np.exp2(rng.integers(-14, 14, (-(-R // 32), -(-C // 32)))).repeat(32, 0).repeat(32, 1)[:R, :C]
        W = O.round_bf16(W)
        q, e = O.quantize_squares_fp8(W)
        assert e.shape == (-(-R // 32), -(-C // 32))
        np.testing.assert_array_equal(O.dequantize_squares_fp8(q, e), _brute_fp8_squares(W))


def test_fp8_squares_of_the_transpose_are_the_transposed_squares():
    """One square quantization serves both read directions: quantizing W^T
    gives W's codes and exponents transposed (ragged shape)."""
    rng = np.random.default_rng(61)
    W = O.round_bf16(rng.standard_normal((75, 130)) * np.exp2(rng.integers(-9, 9, (75, 1))))
    q, e = O.quantize_squares_fp8(W)
    qt, et = O.quantize_squares_fp8(W.T)
    np.testing.assert_array_equal(qt, q.T)
    np.testing.assert_array_equal(et, e.T)


def test_fp8_squares_equal_row_blocks_when_every_row_holds_the_square_max():
    """If every row of every square reaches that square's largest magnitude,
    each 1 x 32 block of a row has the square's scale, so the square codes
    equal quantize_blocks_fp8's and the exponents repeat down the square."""
    rng = np.random.default_rng(62)
    R, C = 64, 96
    W = O.round_bf16(rng.uniform(-1, 1, (R, C)))
    for i0 in range(0, R, 32):
        for j0 in range(0, C, 32):
            s = 2.0 ** int(rng.integers(-10, 10))
            W[i0:i0 + 32, j0:j0 + 32] *= s
            W[i0:i0 + 32, j0 + int(rng.integers(0, 32))] = 1.5 * s * rng.choice([-1.0, 1.0], 32)
    qs, es = O.quantize_squares_fp8(W)
    qb, eb = O.quantize_blocks_fp8(W)
    np.testing.assert_array_equal(qs, qb)
    np.testing.assert_array_equal(es.repeat(32, axis=0), eb)


def test_fp8_squares_share_one_scale_down_the_rows():
    """A square holds one scale for all its rows: a row 2^-17 below the
    square's largest row falls into E4M3's subnormal range and loses its
    precision, where 1 x 32 blocks of its own keep every element within
    2^-4 (so the two schemes are told apart)."""
    rng = np.random.default_rng(63)
    W = O.round_bf16(1.0 + rng.random((32, 32)))
    W[:, 0] = 1.875                              # every row holds the square's largest value
    W[1] *= 2.0 ** -17
    S = O.dequantize_squares_fp8(*O.quantize_squares_fp8(W))
    B = O.dequantize_blocks_fp8(*O.quantize_blocks_fp8(W))
    assert (np.abs(B - W) <= 2.0 ** -4 * np.abs(W) * (1 + 1e-12)).all()
    assert np.abs(S[1] - W[1]).max() > 0.1 * np.abs(W[1]).max()
    np.testing.assert_array_equal(S[[0] + list(range(2, 32))], B[[0] + list(range(2, 32))])


def test_fp8_square_exponent_is_clipped_to_the_scale_range():
    W = np.zeros((64, 32))
    W[:32] = 2.0 ** -140                         # wants 2^-148: clipped to 2^-127
    W[40, 3] = 1.5 * 2.0 ** 100
    q, e = O.quantize_squares_fp8(W)
    assert e.tolist() == [[-127], [92]]
    assert (O.e4m3_decode(q[:32]) == 0).all()


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_expert_forward_fp8_square_brute_force(act):
    """The square-mode forward against explicit loops: X and the bf16 H in
    brute-force 1 x 32 blocks, w13 and w2 in brute-force 32 x 32 squares
    (d = 40, f = 24: partial blocks and squares in both GEMMs)."""
    rng = np.random.default_rng(64)
    n, d, f = 5, 40, 24
    P = 2 * f if act == "swiglu" else f
    X = O.round_bf16(rng.standard_normal((n, d)))
    w13 = O.round_bf16(rng.standard_normal((P, d)) / 6)
    w13[:32, :32] *= 2.0 ** 7                    # squares of different magnitude
    w2 = O.round_bf16(rng.standard_normal((d, f)) / 5)
    w2[32:] *= 2.0 ** -6
    Xd, W13d, W2d = _brute_fp8_blocks(X), _brute_fp8_squares(w13), _brute_fp8_squares(w2)
    pre = np.array([[sum(Xd[t, c] * W13d[j, c] for c in range(d)) for j in range(P)] for t in range(n)])
    if act == "swiglu":
        a, b = pre[:, :f], pre[:, f:]
        H = a / (1 + np.exp(-a)) * b
    else:
        H = 0.5 * pre * (1 + sps.erf(pre / np.sqrt(2)))
    Hd = _brute_fp8_blocks(O.round_bf16(H))
    out = np.array([[sum(Hd[t, j] * W2d[c, j] for j in range(f)) for c in range(d)] for t in range(n)])
    got, saved = O.expert_forward_fp8_square(X, w13, w2, act)
    np.testing.assert_allclose(got, out, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(saved["H"], H, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("act,e5", [("swiglu", False), ("gelu", False), ("swiglu", True)])
def test_expert_backward_fp8_square_brute_force(act, e5):
    """The square-mode data gradients against explicit loops: bf16 dO in
    brute-force 1 x 32 blocks along d, W2 in brute-force squares read along
    its output dimension, the activation backward on the bf16 pre-activations,
    bf16 dpre in 1 x 32 blocks along P, W13 in squares read along P (d = 40,
    P = 48 or 24: partial blocks); gradients in E4M3 or E5M2."""
    rng = np.random.default_rng(65)
    n, d, f = 4, 40, 24
    P = 2 * f if act == "swiglu" else f
    X = O.round_bf16(rng.standard_normal((n, d)))
    w13 = O.round_bf16(rng.standard_normal((P, d)) / 5)
    w13[32:] *= 2.0 ** -5
    w2 = O.round_bf16(rng.standard_normal((d, f)) / 4)
    w2[:, :8] *= 2.0 ** 6
    _, saved = O.expert_forward(X, w13, w2, act)
    dO = rng.standard_normal((n, d)) * 0.3
    dO[:, 32:] *= 2.0 ** -8
    dOd = _brute_fp8_blocks_fmt(O.round_bf16(dO), e5)
    W2d, W13d = _brute_fp8_squares(w2), _brute_fp8_squares(w13)     # [d, f], [P, d]
    dH = np.array([[sum(dOd[t, c] * W2d[c, j] for c in range(d)) for j in range(f)] for t in range(n)])
    a = O.round_bf16(saved["a"])
    sg = 1 / (1 + np.exp(-a))
    if act == "swiglu":
        b = O.round_bf16(saved["b"])
        dpre = np.concatenate([dH * b * sg * (1 + a * (1 - sg)), dH * a * sg], axis=1)
    else:
        cdf = 0.5 * (1 + sps.erf(a / np.sqrt(2)))
        dpre = dH * (cdf + a * np.exp(-a * a / 2) / np.sqrt(2 * np.pi))
    dpd = _brute_fp8_blocks_fmt(O.round_bf16(dpre), e5)
    dX = np.array([[sum(dpd[t, p] * W13d[p, j] for p in range(P)) for j in range(d)] for t in range(n)])
    fmt = "e5m2" if e5 else "e4m3"
    gX, g13, g2, gpre = O.expert_backward_fp8_wq(X, O.quantize_weights_fp8_square(w2).T,
                                                 O.quantize_weights_fp8_square(w13).T, saved, dO, act,
                                                 fmt, "block")
    np.testing.assert_allclose(gpre, dpre, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gX, dX, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g2, dO.T @ saved["H"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g13, dpre.T @ X, rtol=1e-12, atol=1e-14)
    ex, _, _, _ = O.expert_backward(X, w13, w2, saved, dO, act)
    assert np.abs(gX - ex).max() < 0.15 * np.abs(ex).max()


def test_grouped_square_mode_is_per_expert():
    """grouped_ffn_forward(fp8="square") and grouped_ffn_backward(fp8_dgrad=
    "square") run each expert (and the shared one) on its own rows through the
    square-mode expert functions, weights quantized per expert. A few columns
    of w2 sit 2^-12 below the rest: squares round them into E4M3's subnormal
    range, one scale per column would not, so the two weight readings differ."""
    rng = np.random.default_rng(66)
    d, f, E, T = 32, 16, 3, 10
    offsets = np.array([0, 4, 4, 9])
    x = O.round_bf16(rng.standard_normal((T, d)))
    x_perm = x[[0, 2, 5, 7, 1, 3, 4, 8, 9]]
    w13 = O.round_bf16(rng.standard_normal((E, 2 * f, d)) / 3 * np.array([1.0, 2.0 ** 9, 2.0 ** -9])[:, None, None])
    w2 = rng.standard_normal((E, d, f)) / 3
    w2[:, :, :4] *= 2.0 ** -12                   # columns a per-column scale would keep exact
    w2 = O.round_bf16(w2)
    sw13 = O.round_bf16(rng.standard_normal((1, 2 * f, d)) / 3)
    sw2 = O.round_bf16(rng.standard_normal((1, d, f)) / 3)
    O_, Os, saved = O.grouped_ffn_forward(x_perm, offsets, w13, w2, "swiglu", x, sw13, sw2, fp8="square")
    dO = O.round_bf16(rng.standard_normal((9, d)))
    dY = O.round_bf16(rng.standard_normal((T, d)))
    g = O.grouped_ffn_backward(x_perm, offsets, w13, w2, saved, dO, "swiglu", x, sw13, sw2, dY,
                               fp8_dgrad="square")
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        o, sv = O.expert_forward_fp8_square(x_perm[lo:hi], w13[e], w2[e], "swiglu")
        np.testing.assert_array_equal(O_[lo:hi], o)
        dx, _, _, _ = O.expert_backward_fp8_wq(x_perm[lo:hi], O.quantize_weights_fp8_square(w2[e]).T,
                                               O.quantize_weights_fp8_square(w13[e]).T, sv, dO[lo:hi],
                                               "swiglu", "e4m3", "block")
        np.testing.assert_array_equal(g["dx_perm"][lo:hi], dx)
    os_, svs = O.expert_forward_fp8_square(x, sw13[0], sw2[0], "swiglu")
    np.testing.assert_array_equal(Os, os_)
    dxs, _, _, _ = O.expert_backward_fp8_wq(x, O.quantize_weights_fp8_square(sw2[0]).T,
                                            O.quantize_weights_fp8_square(sw13[0]).T, svs, dY, "swiglu",
                                            "e4m3", "block")
    np.testing.assert_array_equal(g["dx_shared"], dxs)
    per_col = O.grouped_ffn_backward(x_perm, offsets, w13, w2, saved, dO, "swiglu", x, sw13, sw2, dY,
                                     fp8_dgrad=True)
    assert (per_col["dx_perm"] != g["dx_perm"]).any()
