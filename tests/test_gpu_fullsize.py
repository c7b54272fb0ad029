"""Full-size parity of the benchmarked workload (Mixtral-like layer, bf16:
T=8192, d=4096, E=8, k=2, SwiGLU f=14336, capacity factor 1.25), launched
exactly as bench.py launches it. The oracle checks the whole router,
statistics and permutation, and sampled tokens / sampled hidden columns of
the FFN outputs and gradients, computed one by one with the oracle's own
functions (the expert FFN is separable over hidden columns, so columns J of
dW2 and rows J, f+J of dW13 come from the oracle run on those columns only).
"""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import WORKLOADS, as_f64, gen_all
from parity_util import Report, assert_close, bits, gpu_layer, to_np

pytestmark = pytest.mark.gpu


def check_sampled(w, n_tok=24, n_exp=2, n_col=4, seed=123):
    print(f"[case] full size {w}", flush=True)
    g = gen_all(w)
    L, dev = gpu_layer(w, g)
    print("[step] gpu layer done", flush=True)
    rep = Report()
    dt = w.dtype
    x = as_f64(g["x"], dt)
    dy = as_f64(g["dy"], dt)
    w_r = g["w_r"].astype(np.float64)
    lb = g["logit_bias"].astype(np.float64) if g["logit_bias"] is not None else None
    sb = g["sel_bias"].astype(np.float64) if g["sel_bias"] is not None else None
    r = O.router_forward(x, w_r, w.k, w.score, lb, sb)
    st = O.aux_stats(r["scores"], r["topk_idx"], w.E)
    cap = O.capacity(w.T, w.k, w.E, w.cf)
    pm = O.permute(r["topk_idx"], w.E, cap)
    # ---- whole router / stats / permute
    g_idx = L.topk_idx.cpu().numpy().astype(np.int64)
    flagged = O.near_tie_tokens(r["key"], w.k)
    diff = (g_idx != r["topk_idx"]).any(axis=1)
    assert not (diff & ~flagged).any()
    rep.add("routing", flagged=int(flagged.sum()), flips=int(diff.sum()))
    assert not diff.any(), "a near-tie flipped at full size; sampled checks assume none"
    assert_close("scores", to_np(L.scores), r["scores"], dt, rep, rel=1e-5)
    assert_close("gate", to_np(L.gate), r["gates"], dt, rep, rel=1e-5)
    assert (L.counts.cpu().numpy() == st["counts"]).all()
    assert_close("z", to_np(L.z_mean), st["z"], dt, rep, rel=1e-5)
    assert_close("lse", to_np(L.lse), O.router_logsumexp(r["logits"]), dt, rep, rel=1e-5)
    assert_close("S,L_aux,L_z", to_np(L.aux_out),
                 np.array([st["S"], st["L_aux"], O.z_loss(r["logits"])]), dt, rep, rel=1e-5)
    off = L.offsets.cpu().numpy().astype(np.int64)
    assert (off == pm["offsets"]).all()
    assert int(L.n_dropped.cpu()[0]) == pm["n_dropped"]
    assert (L.row_of.cpu().numpy() == pm["row_of"]).all()
    A = int(off[-1])
    tok = L.token_of.cpu().numpy()[:A]
    assert (tok == pm["token_of"]).all()
    assert (bits(L.x_perm)[:A] == bits(dev["x"])[tok]).all()
    rep.add("permute", rows=A, dropped=pm["n_dropped"])
    print("[step] router/permute checked", flush=True)

    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(w.T, size=n_tok, replace=False))
    gate = r["gates"]
    g_O, g_H, g_pre = to_np(L.out), to_np(L.save_h), to_np(L.save_pre)
    g_dO, g_dxp = to_np(L.dout), to_np(L.dx_perm)
    ref = {k_: [] for k_ in ("O", "H", "pre", "dO", "dxp")}
    got = {k_: [] for k_ in ref}
    Y_ref = np.zeros((n_tok, w.d))
    dX_ref = np.zeros((n_tok, w.d))
    dgate_ref = np.zeros((n_tok, w.k))
    exps = sorted(set(rng.choice(w.E, size=n_exp, replace=False).tolist()))
    dw13_ref, dw2_ref, dw13_got, dw2_got = [], [], [], []
    g_dw13, g_dw2 = L.dw13, L.dw2
    for e in range(w.E):
        w13e = as_f64(g["w13"][e], dt)
        w2e = as_f64(g["w2"][e], dt)
        # sampled tokens routed to e
        for i, t in enumerate(toks):
            for j in range(w.k):
                if r["topk_idx"][t, j] != e or pm["row_of"][t, j] < 0:
                    continue
                row = pm["row_of"][t, j]
                o, sv = O.expert_forward(x[t:t + 1], w13e, w2e, w.act)
                pre = np.concatenate([sv["a"], sv["b"]], 1) if w.act == "swiglu" else sv["a"]
                dgate_ref[i, j] = float(dy[t] @ o[0])
                dO = gate[t, j] * dy[t:t + 1]
                dxr, _, _, _ = O.expert_backward(x[t:t + 1], w13e, w2e, sv, dO, w.act)
                Y_ref[i] += gate[t, j] * o[0]
                dX_ref[i] += dxr[0]
                ref["O"].append(o[0]); got["O"].append(g_O[row])
                ref["H"].append(sv["H"][0]); got["H"].append(g_H[row])
                ref["pre"].append(pre[0]); got["pre"].append(g_pre[row])
                ref["dO"].append(dO[0]); got["dO"].append(g_dO[row])
                ref["dxp"].append(dxr[0]); got["dxp"].append(g_dxp[row])
        if e in exps:
            lo, hi = pm["offsets"][e], pm["offsets"][e + 1]
            rows_t = pm["token_of"][lo:hi]
            slot = np.array([int(np.nonzero(r["topk_idx"][t] == e)[0][0]) for t in rows_t])
            Xe = x[rows_t]
            dOe = gate[rows_t, slot][:, None] * dy[rows_t]
            J = np.sort(rng.choice(w.f, size=n_col, replace=False))
            rows13 = np.concatenate([J, w.f + J]) if w.act == "swiglu" else J
            _, sv = O.expert_forward(Xe, w13e[rows13], w2e[:, J], w.act)
            _, d13, d2, _ = O.expert_backward(Xe, w13e[rows13], w2e[:, J], sv, dOe, w.act)
            dw13_ref.append(d13)
            dw2_ref.append(d2)
            dw13_got.append(to_np(g_dw13[e][torch.as_tensor(rows13, device="cuda")]))
            dw2_got.append(to_np(g_dw2[e][:, torch.as_tensor(J, device="cuda")]))
        del w13e, w2e
    print("[step] sampled oracle done", flush=True)
    for k_ in ref:
        assert_close(k_, np.array(got[k_]), np.array(ref[k_]), dt, rep)
    # router backward of the sampled tokens, then Y / dgate / dX rows
    rb = O.router_backward(x[toks], w_r, r["scores"][toks], r["topk_idx"][toks], gate[toks],
                           dgate_ref, w.score, w.aux_coef, st["y"])
    dX_ref += rb["dx_router"]
    assert_close("Y", to_np(L.Y)[toks], Y_ref, dt, rep)
    assert_close("dgate", to_np(L.dgate)[toks], dgate_ref, dt, rep)
    assert_close("dlogits", to_np(L.dlogits)[toks], rb["dlogits"], dt, rep)
    assert_close("dX", to_np(L.dX)[toks], dX_ref, dt, rep)
    assert_close("dW13[sampled]", np.array(dw13_got), np.array(dw13_ref), dt, rep)
    assert_close("dW2[sampled]", np.array(dw2_got), np.array(dw2_ref), dt, rep)
    gdl = to_np(L.dlogits)
    assert_close("dW_r(own dl)", to_np(L.dw_r), gdl.T @ x, dt, rep, rel=2e-5)
    print(rep, flush=True)


def test_fullsize_mixtral_sampled():
    check_sampled(WORKLOADS["mixtral_bf16"])
