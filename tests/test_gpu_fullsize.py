"""Full-size parity of every layer configuration, launched exactly as bench.py
launches it (same workload presets, same layer object, one fwd+bwd step):

  mixtral_bf16      T=8192  d=4096 E=8   k=2 SwiGLU f=14336, cf 1.25
  skewed_bf16       T=4096  d=4096 E=8   k=2 GELU f=16384, logit bias, cf 1.0
  skewed_nocap_bf16 the same without a capacity limit
  finegrained_bf16  T=16384 d=4096 E=128 k=8 SwiGLU f=1536, aux 0.01, z-loss 1e-3
  dsv3_bf16         T=8192  d=7168 E=256 k=8 sigmoid + selection bias (and its
                    update), one shared expert, SwiGLU f=2048
  mixtral_fp8_bf16  the Mixtral-like layer with FP8 (E4M3) forward GEMMs
  mixtral_fp8_dgrad_bf16  the same with FP8 data-gradient GEMMs as well
  mixtral_fp8b_bf16 the Mixtral-like layer with block-scaled FP8 forward GEMMs
                    (one scale per 32 elements along K)
  mixtral_fp8_all_bf16 every GEMM on FP8 operands (weight gradients with
                    token-axis block scales)
  mixtral_fp8_all_e5m2_bf16 the same with E5M2 gradient operands
  mixtral_fp8sq_all_bf16 every GEMM on FP8 operands with 32 x 32 weight
                    squares (forward and data gradients on block scales)

The oracle checks the whole router, statistics and permutation, and sampled
tokens / sampled hidden columns of the FFN outputs and gradients, computed
one by one with the oracle's own functions (the expert FFN is separable over
hidden columns, so columns J of dW2 and rows J, f+J of dW13 come from the
oracle run on those columns only). Tokens whose fp32 routing legitimately
differs from the oracle's at a near-tie are excluded, with the experts they
touch, as in the reduced-size tests.
"""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import WORKLOADS, as_f64, gen_all
from parity_util import (Report, assert_close, assert_rows_match, bits, fp8_dgrad_tol, fp8_wgrad_tol,
                         gpu_layer, to_np)

pytestmark = pytest.mark.gpu


def check_sampled(w, n_tok=24, n_exp=2, n_col=4, seed=123, expert_subset=None):
    """expert_subset: sample only tokens routed entirely to these experts (and
    weight-gradient columns of them), so that the oracle quantizes only their
    weights."""
    print(f"[case] full size {w}", flush=True)
    g = gen_all(w)
    L, dev = gpu_layer(w, g)
    print("[step] gpu layer done", flush=True)
    rep = Report()
    dt = w.dtype
    T, k, E = w.T, w.k, w.E
    x = as_f64(g["x"], dt)
    dy = as_f64(g["dy"], dt)
    w_r = g["w_r"].astype(np.float64)
    lb = g["logit_bias"].astype(np.float64) if g["logit_bias"] is not None else None
    sb = g["sel_bias"].astype(np.float64) if g["sel_bias"] is not None else None
    r = O.router_forward(x, w_r, k, w.score, lb, sb)
    st = O.aux_stats(r["scores"], r["topk_idx"], E)
    cap = O.capacity(T, k, E, w.cf)
    pm = O.permute(r["topk_idx"], E, cap)
    # ---- whole router / stats / permute; near-tie flips are valid and excluded
    g_idx = L.topk_idx.cpu().numpy().astype(np.int64)
    flagged = O.near_tie_tokens(r["key"], k)
    diff = (g_idx != r["topk_idx"]).any(axis=1)
    assert not (diff & ~flagged).any(), "routing differs at unflagged tokens"
    bad_e = set()
    for t in np.nonzero(diff)[0]:
        kth = np.sort(r["key"][t])[::-1][k - 1]
        assert (r["key"][t, g_idx[t]] >= kth - 2 * O.NEAR_TIE).all()
        bad_e |= set(g_idx[t].tolist()) ^ set(r["topk_idx"][t].tolist())
    tok_ok = ~diff
    if bad_e and w.cf is not None:   # capacity ranks shift inside affected experts
        for e in bad_e:
            tok_ok &= ~(r["topk_idx"] == e).any(axis=1)
            tok_ok &= ~(g_idx == e).any(axis=1)
    e_ok = np.array([e not in bad_e for e in range(E)])
    rep.add("routing", flagged=int(flagged.sum()), flips=int(diff.sum()), bad_experts=len(bad_e))
    assert_close("scores", to_np(L.scores), r["scores"], dt, rep, rel=1e-5)
    assert_close("gate", to_np(L.gate)[tok_ok], r["gates"][tok_ok], dt, rep, rel=1e-5)
    counts = L.counts.cpu().numpy()
    assert (counts[e_ok] == st["counts"][e_ok]).all()
    assert counts.sum() == T * k
    assert_close("z", to_np(L.z_mean), st["z"], dt, rep, rel=1e-5)
    assert_close("lse", to_np(L.lse), O.router_logsumexp(r["logits"]), dt, rep, rel=1e-5)
    if not bad_e:
        assert_close("S,L_aux,L_z", to_np(L.aux_out),
                     np.array([st["S"], st["L_aux"], O.z_loss(r["logits"])]), dt, rep, rel=1e-5)
        if w.bias_gamma and sb is not None:
            assert_close("sel_bias update", to_np(dev["sel_bias"]),
                         O.bias_update(sb, st["counts"], T, k, w.bias_gamma), dt, rep, rel=1e-6)
    off = L.offsets.cpu().numpy().astype(np.int64)
    A = int(off[-1])
    tok = L.token_of.cpu().numpy()[:A]
    if not bad_e:
        assert (off == pm["offsets"]).all()
        assert int(L.n_dropped.cpu()[0]) == pm["n_dropped"]
        assert_rows_match(g_idx, L.row_of.cpu().numpy(), r["topk_idx"], pm["row_of"])
        assert (tok == pm["token_of"]).all()
    assert (bits(L.x_perm)[:A] == bits(dev["x"])[tok]).all()
    rep.add("permute", rows=A, dropped=T * k - A)
    print("[step] router/permute checked", flush=True)

    rng = np.random.default_rng(seed)
    # sampled tokens: routed entirely to unaffected experts and not flipped
    allowed = e_ok.copy()
    if expert_subset is not None:
        allowed &= np.isin(np.arange(E), expert_subset)
    cand = np.nonzero(tok_ok & allowed[r["topk_idx"]].all(axis=1))[0]
    assert len(cand) > 0, "no token routed entirely to the sampled experts"
    toks = np.sort(rng.choice(cand, size=min(n_tok, len(cand)), replace=False))
    exps = sorted(set(rng.choice(np.nonzero(allowed)[0], size=min(n_exp, int(allowed.sum())),
                                 replace=False).tolist()))
    gate = r["gates"]
    g_row_of = L.row_of.cpu().numpy()
    # routed buffers hold T*k rows; only the first A are written
    g_O, g_H, g_pre = to_np(L.out[:A]), to_np(L.save_h[:A]), to_np(L.save_pre[:A])
    g_dO, g_dxp = to_np(L.dout[:A]), to_np(L.dx_perm[:A])
    ref = {k_: [] for k_ in ("O", "H", "pre", "dO", "dxp")}
    got = {k_: [] for k_ in ref}
    n = len(toks)
    Y_ref = np.zeros((n, w.d))
    dX_ref = np.zeros((n, w.d))
    dgate_ref = np.zeros((n, k))
    dw13_ref, dw2_ref, dw13_got, dw2_got = [], [], [], []
    sampled_e = set(r["topk_idx"][toks].ravel().tolist())
    # FP8 forward: per-row quantization, so single rows and weight-row subsets
    # quantize exactly as in the whole GEMM; each expert's weights are
    # quantized once (w13d, w2d) and sliced like the bf16 ones
    # (block scales: the same holds, blocks run along a row)
    # (square-block weights: each expert's weight is quantized whole, then
    # sliced; both GEMM directions read the same dequantized matrix)
    blk = w.fp8 and w.fp8_scale == "block"
    sq = w.fp8_scale == "square"

    def wq(m):
        if not w.fp8:
            return m
        if sq:
            return O.quantize_weights_fp8_square(m)
        return O.quantize_weights_fp8_block(m) if blk else O.quantize_weights_fp8(m)
    efwd = (O.expert_forward_fp8_block_wq if blk or sq else O.expert_forward_fp8_wq) if w.fp8 \
        else O.expert_forward
    # FP8 data gradients: the weights quantized per input channel (rows of the
    # transpose), once per expert; any subset of those rows quantizes the same
    # way, and a token row's dO and dpre are quantized on their own.
    def ebwd(X, w13e, w2e, w13t, w2t, sv, dO):
        if w.fp8_bwd:
            return O.expert_backward_fp8_wq(X, w2t, w13t, sv, dO, w.act, w.fp8_grad,
                                            "block" if sq else "row")
        return O.expert_backward(X, w13e, w2e, sv, dO, w.act)

    def wq_t(m):
        if not w.fp8_bwd:
            return None
        return O.quantize_weights_fp8_square(m).T if sq else O.quantize_weights_fp8_t(m)
    dxt = fp8_dgrad_tol(w.f, w.fp8_grad) if w.fp8_bwd else {}
    # FP8 weight gradients: the bound of the smallest sampled expert's rows
    nrows = [int(pm["offsets"][e + 1] - pm["offsets"][e]) for e in exps]
    wgt = fp8_wgrad_tol(min([n for n in nrows if n > 0], default=w.T), w.fp8_grad) if w.fp8_wgrad else {}
    wgt_s = fp8_wgrad_tol(w.T, w.fp8_grad) if w.fp8_wgrad else {}
    for e in range(E):
        if e not in sampled_e and e not in exps:
            continue
        print(f"[step] oracle expert {e}", flush=True)
        w13e = as_f64(g["w13"][e], dt)
        w2e = as_f64(g["w2"][e], dt)
        w13f, w2f = wq(w13e), wq(w2e)   # the forward's weights (FP8-quantized when w.fp8)
        w13t, w2t = wq_t(w13e), wq_t(w2e)
        for i, t in enumerate(toks):
            for j in range(k):
                if r["topk_idx"][t, j] != e or pm["row_of"][t, j] < 0:
                    continue
                row = g_row_of[t, j]
                o, sv = efwd(x[t:t + 1], w13f, w2f, w.act)
                pre = np.concatenate([sv["a"], sv["b"]], 1) if w.act == "swiglu" else sv["a"]
                dgate_ref[i, j] = float(dy[t] @ o[0])
                dO = gate[t, j] * dy[t:t + 1]
                dxr, _, _, _ = ebwd(x[t:t + 1], w13e, w2e, w13t, w2t, sv, dO)
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
            slot = np.array([int(np.nonzero(r["topk_idx"][t] == e)[0][0]) for t in rows_t],
                            dtype=np.int64)
            Xe = x[rows_t]
            dOe = gate[rows_t, slot][:, None] * dy[rows_t]
            J = np.sort(rng.choice(w.f, size=n_col, replace=False))
            rows13 = np.concatenate([J, w.f + J]) if w.act == "swiglu" else J
            _, sv = efwd(Xe, w13f[rows13], w2f[:, J], w.act)
            # hidden columns J only: dH[:, J] needs rows J of w2's transpose
            # (dX of this call is not used: it would need all of dpre's row)
            _, d13, d2, dpc = ebwd(Xe, w13e[rows13], w2e[:, J],
                                   None if w13t is None else w13t[:, rows13],
                                   None if w2t is None else w2t[J], sv, dOe)
            if w.fp8_wgrad:   # per-column token-axis quantization: columns separate
                d13, d2 = O.expert_wgrad_fp8(Xe, sv["H"], dOe, dpc, w.fp8_grad)
            dw13_ref.append(d13)
            dw2_ref.append(d2)
            dw13_got.append(to_np(L.dw13[e][torch.as_tensor(rows13, device="cuda")]))
            dw2_got.append(to_np(L.dw2[e][:, torch.as_tensor(J, device="cuda")]))
        del w13e, w2e, w13f, w2f, w13t, w2t
    if w.n_shared:
        # the shared expert: sampled tokens' outputs and input gradients, and
        # sampled hidden columns of its weight gradients over all tokens
        sw13 = as_f64(g["sw13"][0], dt)
        sw2 = as_f64(g["sw2"][0], dt)
        sw13f, sw2f = wq(sw13), wq(sw2)
        sw13t, sw2t = wq_t(sw13), wq_t(sw2)
        os_, svs = efwd(x[toks], sw13f, sw2f, w.act)
        dxs, _, _, _ = ebwd(x[toks], sw13, sw2, sw13t, sw2t, svs, dy[toks])
        Y_ref += os_
        dX_ref += dxs
        assert_close("O_shared", to_np(L.out_shared)[toks], os_, dt, rep)
        assert_close("dX_shared", to_np(L.dx_shared)[toks], dxs, dt, rep, **dxt)
        J = np.sort(rng.choice(w.f, size=n_col, replace=False))
        rows13 = np.concatenate([J, w.f + J]) if w.act == "swiglu" else J
        _, sv = efwd(x, sw13f[rows13], sw2f[:, J], w.act)
        _, d13, d2, dpc = ebwd(x, sw13[rows13], sw2[:, J],
                               None if sw13t is None else sw13t[:, rows13],
                               None if sw2t is None else sw2t[J], sv, dy)
        if w.fp8_wgrad:
            d13, d2 = O.expert_wgrad_fp8(x, sv["H"], dy, dpc, w.fp8_grad)
        assert_close("dSW13[sampled]", to_np(L.dsw13[0][torch.as_tensor(rows13, device="cuda")]),
                     d13, dt, rep, **wgt_s)
        assert_close("dSW2[sampled]", to_np(L.dsw2[0][:, torch.as_tensor(J, device="cuda")]), d2,
                     dt, rep, **wgt_s)
        del sw13, sw2
    print("[step] sampled oracle done", flush=True)
    for k_ in ref:
        assert_close(k_, np.array(got[k_]), np.array(ref[k_]), dt, rep,
                     **(dxt if k_ == "dxp" else {}))
    # router backward of the sampled tokens (batch-wide 1/T factors), then Y / dgate / dX rows
    rb = O.router_backward(x[toks], w_r, r["scores"][toks], r["topk_idx"][toks], gate[toks],
                           dgate_ref, w.score, w.aux_coef, st["y"], w.z_coef, r["logits"][toks],
                           n_tokens=T)
    dX_ref += rb["dx_router"]
    assert_close("Y", to_np(L.Y)[toks], Y_ref, dt, rep)
    assert_close("dgate", to_np(L.dgate)[toks], dgate_ref, dt, rep)
    dl_floor = 2e-6 * float(np.abs(dgate_ref).max(initial=0.0))
    assert_close("dlogits", to_np(L.dlogits)[toks], rb["dlogits"], dt, rep, atol=dl_floor)
    assert_close("dX", to_np(L.dX)[toks], dX_ref, dt, rep, **dxt)
    if dw13_ref:
        assert_close("dW13[sampled]", np.array(dw13_got), np.array(dw13_ref), dt, rep, **wgt)
        assert_close("dW2[sampled]", np.array(dw2_got), np.array(dw2_ref), dt, rep, **wgt)
    gdl = to_np(L.dlogits)
    assert_close("dW_r(own dl)", to_np(L.dw_r), gdl.T @ x, dt, rep, rel=2e-5)
    # the whole router backward against the oracle's, on every token, given
    # the GPU's own routing and dgate (the GPU may list a token's two
    # near-tied experts in the other slot order; its dgate follows its own
    # order), with the oracle's scores and logits
    if not bad_e:
        g_dgate = to_np(L.dgate)
        rb_all = O.router_backward(x, w_r, r["scores"], g_idx, to_np(L.gate), g_dgate, w.score,
                                   w.aux_coef, st["y"], w.z_coef, r["logits"])
        floor_all = 2e-6 * float(np.abs(g_dgate).max(initial=0.0))
        assert_close("dlogits(own dgate, all tokens)", gdl, rb_all["dlogits"], dt, rep,
                     atol=floor_all)
        assert_close("dW_r(own dgate)", to_np(L.dw_r), rb_all["dw_r"], dt, rep,
                     atol=floor_all * float(np.abs(x).sum(axis=0).max(initial=0.0)))
    print(rep, flush=True)
    del L, dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["mixtral_bf16", "skewed_bf16", "skewed_nocap_bf16",
                                  "finegrained_bf16", "dsv3_bf16", "mixtral_fp8_bf16",
                                  "mixtral_fp8_dgrad_bf16", "mixtral_fp8b_bf16", "mixtral_fp8_all_bf16",
                                  "mixtral_fp8_all_e5m2_bf16", "mixtral_fp8sq_all_bf16"])
def test_fullsize_sampled(name):
    w = WORKLOADS[name]
    # the oracle's FP8 backward quantizes each sampled expert's weights both
    # ways (about 45 s per Mixtral-like expert on the host), and its block
    # quantizer walks the weights block by block: two experts
    slow = w.fp8_bwd or w.fp8_scale in ("block", "square")
    check_sampled(w, expert_subset=(2, 5) if slow else None)
