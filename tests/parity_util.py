"""Shared parity helpers: run the layer through libmoe on the GPU and through
the CPU oracle on the same seeded inputs, then compare stage by stage.

Tolerances:
  * integers (routing, counts, offsets, row maps, token maps): bit-exact,
    except tokens the oracle flags as near-ties (adjacent top-(k+1) fp32
    scores closer than 1e-5), where a flip is counted, checked for validity
    and excluded downstream;
  * x_perm: bitwise (a copy);
  * float32 router outputs (scores, gates, lse, z, S, L_aux, L_z, updated
    selection bias): max|d| <= 1e-5 max|ref|;
  * fp32 layer: every float output max|d| <= 1e-5 max|ref|;
  * bf16 layer: max|d| <= 2e-2 max|ref| and sum|d| / sum|ref| <= 5e-3;
  * router gradients (dlogits, dW_r) also get an absolute floor of
    2e-6 max|dgate| (times the largest column sum of |x| for dW_r): with top-1
    routing the exact gradient is identically zero and the GPU holds only
    fp32 rounding of g (1 - g) dg.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from moe_inputs import Workload, as_f64, gen_all


# ----------------------------------------------------------- conversions
def to_dev(a, device="cuda"):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_np(t):
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    if t.dtype in (torch.float32, torch.float64):
        return t.cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def bits(t):
    """Raw bits of a device tensor (for bitwise comparisons)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.cpu().numpy().view(np.int32)


# -------------------------------------------------------------- runners
def oracle_fp8(w: Workload):
    """The oracle's fp8 argument for a workload: False, True (per-row scales),
    "block" or "square"."""
    if not w.fp8:
        return False
    return w.fp8_scale if w.fp8_scale in ("block", "square") else True


def oracle_fp8_dgrad(w: Workload):
    """The oracle's fp8_dgrad argument: False, True (per-row) or "square"."""
    if not w.fp8_bwd:
        return False
    return "square" if w.fp8_scale == "square" else True


def block_bytes(buf, rows, K):
    """[rows, 4 * ceil(K / 128)] bytes (row, block) out of the 32-row
    interleaved scale array: word w of row r is word (r // 32 * KW + w) * 32
    + r % 32, its byte j the scale of block 4w + j."""
    KW = -(-K // 128)
    words = np.asarray(buf, dtype=np.uint8).view("<u4")
    r = np.arange(rows)[:, None]
    w = np.arange(KW)[None, :]
    sel = words[(r // 32 * KW + w) * 32 + r % 32]                      # [rows, KW]
    return ((sel[:, :, None] >> (8 * np.arange(4, dtype=np.uint32))) & 0xFF).reshape(rows, 4 * KW)


def decode_block_codes(codes, scales, row0=0):
    """Dequantized rows of device E4M3 codes [n, K] whose block-scale bytes
    are rows row0 .. row0+n-1 of the interleaved array scales."""
    c = codes.cpu()
    n, K = c.shape
    v = c.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    b = block_bytes(scales.cpu().numpy(), row0 + n, K)[row0:, : -(-K // 32)].astype(np.float64)
    return v * np.repeat(np.exp2(b - 127.0), 32, axis=1)[:, :K]


def gpu_layer(w: Workload, g: dict):
    import mixture_experts_layer_28_amd as moe
    cap = moe.capacity(w.T, w.k, w.E, w.cf)
    L = moe.MoELayer(w.T, w.d, w.E, w.k, w.f, w.n_shared, w.dtype, w.score, w.act, cap,
                     w.aux_coef, w.z_coef, w.bias_gamma, w.gumbel_tau or 0.0, fp8_fwd=w.fp8,
                     fp8_bwd=w.fp8_bwd, fp8_scale=w.fp8_scale, fp8_wgrad=w.fp8_wgrad,
                     fp8_grad=w.fp8_grad)
    dev = {n: to_dev(v) for n, v in g.items()}
    L.step(dev)
    torch.cuda.synchronize()
    return L, dev


def oracle_layer(w: Workload, g: dict):
    f = {n: as_f64(v, w.dtype) for n, v in g.items()}
    cap = O.capacity(w.T, w.k, w.E, w.cf)
    fwd = O.layer_forward(f["x"], f["w_r"], f["w13"], f["w2"], w.k, w.score, w.act, cap,
                          f["logit_bias"], f["sel_bias"], f["sw13"], f["sw2"], f["gumbel_u"],
                          w.gumbel_tau, fp8=oracle_fp8(w))
    bwd = O.layer_backward(fwd, f["x"], f["w_r"], f["w13"], f["w2"], f["dy"], w.score, w.act,
                           w.aux_coef, f["sw13"], f["sw2"], w.z_coef, w.gumbel_tau,
                           fp8_dgrad=oracle_fp8_dgrad(w), fp8_wgrad=w.fp8_wgrad, fp8_grad=w.fp8_grad)
    return fwd, bwd, f


# -------------------------------------------------------------- checks
class Report:
    def __init__(self):
        self.lines = []

    def add(self, name, **kv):
        self.lines.append((name, kv))

    def __str__(self):
        return "\n".join(f"{n}: " + " ".join(f"{k}={v}" for k, v in kv.items())
                         for n, kv in self.lines)


def assert_close(name, got, ref, dtype, rep: Report, rel=None, atol=0.0, max_rel=2e-2, l1_rel=5e-3):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if ref.size == 0:
        return
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = np.abs(got - ref)
    mx = float(np.abs(ref).max())
    l1 = float(err.sum() / max(np.abs(ref).sum(), 1e-300))
    emax = float(err.max())
    rep.add(name, max_err=f"{emax:.3e}", max_ref=f"{mx:.3e}", rel_max=f"{emax / max(mx, 1e-300):.2e}",
            l1_rel=f"{l1:.2e}")
    if rel is not None or dtype == "fp32":
        r = rel if rel is not None else 1e-5
        assert emax <= r * mx + atol + 1e-30, f"{name}: max|d| {emax:.3e} > {r} * {mx:.3e} + {atol:.1e}"
    else:
        assert emax <= max_rel * mx + atol + 1e-30, \
            f"{name}: max|d| {emax:.3e} > {max_rel} * {mx:.3e} + {atol:.1e}"
        if atol == 0.0 or mx > 1e3 * atol:
            assert l1 <= l1_rel, f"{name}: mean relative error {l1:.3e} > {l1_rel}"


def assert_rows_match(g_idx, g_row_of, o_idx, o_row_of):
    """row_of keyed by (token, expert), not by slot: a token whose two
    selected experts sit at a near-tie may list them in either order on the
    two sides while selecting the same set and getting the same rows."""
    go = np.argsort(g_idx, axis=1, kind="stable")
    oo = np.argsort(o_idx, axis=1, kind="stable")
    ge, oe = np.take_along_axis(g_idx, go, 1), np.take_along_axis(o_idx, oo, 1)
    assert (ge == oe).all(), "selected expert sets differ"
    gr = np.take_along_axis(np.asarray(g_row_of, np.int64), go, 1)
    orr = np.take_along_axis(np.asarray(o_row_of, np.int64), oo, 1)
    assert (gr == orr).all(), "row_of differs"


def compare_layer(w: Workload, L, dev, fwd, bwd, f, rep: Report):
    """Stage-by-stage comparison of one fwd+bwd. Returns the number of
    near-tie flips (tokens whose GPU routing differs from the oracle's)."""
    T, k, E, dt = w.T, w.k, w.E, w.dtype
    r, st, pm = fwd["router"], fwd["stats"], fwd["perm"]
    # ---- routing (integer): bit-exact except at flagged near-ties
    g_idx = L.topk_idx.cpu().numpy().astype(np.int64)
    flagged = O.near_tie_tokens(r["key"], k)
    diff = (g_idx != r["topk_idx"]).any(axis=1)
    assert not (diff & ~flagged).any(), \
        f"routing differs at unflagged tokens {np.nonzero(diff & ~flagged)[0][:10]}"
    flips = np.nonzero(diff)[0]
    for t in flips:   # a flipped token must still pick near-maximal keys
        kth = np.sort(r["key"][t])[::-1][k - 1]
        assert (r["key"][t, g_idx[t]] >= kth - 2 * O.NEAR_TIE).all()
        assert len(set(g_idx[t].tolist())) == k
    rep.add("routing", tokens=T, flagged=int(flagged.sum()), flips=len(flips))
    bad_e = set()
    for t in flips:
        bad_e |= set(g_idx[t].tolist()) ^ set(r["topk_idx"][t].tolist())
    tok_ok = ~diff
    if bad_e and w.cf is not None:   # capacity ranks shift inside affected experts
        for e in bad_e:
            tok_ok &= ~(r["topk_idx"] == e).any(axis=1)
            tok_ok &= ~(g_idx == e).any(axis=1)
    e_ok = np.array([e not in bad_e for e in range(E)])

    assert_close("scores", to_np(L.scores), r["scores"], dt, rep, rel=1e-5)
    lse_ref = O.router_logsumexp(r["logits"])
    assert_close("lse", to_np(L.lse), lse_ref, dt, rep, rel=1e-5)
    assert_close("gate", to_np(L.gate)[tok_ok], r["gates"][tok_ok], dt, rep, rel=1e-5)
    # ---- stats
    counts = L.counts.cpu().numpy()
    assert (counts[e_ok] == st["counts"][e_ok]).all(), "expert counts differ"
    assert counts.sum() == T * k
    assert_close("y", to_np(L.y_frac)[e_ok], st["y"][e_ok], dt, rep, rel=1e-6)
    assert_close("z", to_np(L.z_mean), st["z"], dt, rep, rel=1e-5)
    if not bad_e:
        aux = to_np(L.aux_out)
        assert_close("S,L_aux,L_z", aux, np.array([st["S"], st["L_aux"], O.z_loss(r["logits"])]),
                     dt, rep, rel=1e-5)
    if w.bias_gamma and f.get("sel_bias") is not None and not bad_e:
        ref_b = O.bias_update(f["sel_bias"], st["counts"], T, k, w.bias_gamma)
        assert_close("sel_bias update", to_np(dev["sel_bias"]), ref_b, dt, rep, rel=1e-6)
    # ---- permute (integer, bitwise copy)
    off = L.offsets.cpu().numpy().astype(np.int64)
    A = int(off[-1])
    nd = int(L.n_dropped.cpu().numpy()[0])
    assert A + nd == T * k
    row_of = L.row_of.cpu().numpy().astype(np.int64)
    token_of = L.token_of.cpu().numpy().astype(np.int64)[:A]
    if not bad_e:
        assert (off == pm["offsets"]).all(), "offsets differ"
        assert nd == pm["n_dropped"]
        assert_rows_match(g_idx, row_of, r["topk_idx"], pm["row_of"])
        assert (token_of == pm["token_of"]).all(), "token_of differs"
    xb = bits(dev["x"])
    xpb = bits(L.x_perm)[:A]
    assert (xpb == xb[token_of]).all(), "x_perm is not x[token_of]"
    rep.add("permute", rows=A, dropped=nd)
    # rows of experts untouched by flips: same tokens in the same order on
    # both sides, only shifted by the other experts' counts
    g_rows, o_rows = [], []
    for e in range(E):
        if e_ok[e]:
            n = int(off[e + 1] - off[e])
            assert n == pm["offsets"][e + 1] - pm["offsets"][e]
            g_rows.append(np.arange(off[e], off[e] + n))
            o_rows.append(np.arange(pm["offsets"][e], pm["offsets"][e] + n))
    g_rows = np.concatenate(g_rows).astype(np.int64) if g_rows else np.zeros(0, np.int64)
    o_rows = np.concatenate(o_rows).astype(np.int64) if o_rows else np.zeros(0, np.int64)
    # ---- grouped FFN forward
    P = 2 * w.f if w.act == "swiglu" else w.f
    Ao = int(pm["offsets"][-1])
    if Ao:
        pre_ref = np.concatenate(
            [np.concatenate([s["a"], s["b"]], axis=1) if w.act == "swiglu" else s["a"]
             for s in fwd["saved"]["routed"]], axis=0)
        h_ref = np.concatenate([s["H"] for s in fwd["saved"]["routed"]], axis=0)
    else:
        pre_ref, h_ref = np.zeros((0, P)), np.zeros((0, w.f))
    assert_close("pre(a|b)", to_np(L.save_pre[:A])[g_rows], pre_ref[o_rows], dt, rep)
    assert_close("H", to_np(L.save_h[:A])[g_rows], h_ref[o_rows], dt, rep)
    # FP8 forward: H is quantized from its stored bf16 value on both sides, and
    # the two sides' bf16 H can differ in the last bit (float32 vs float64
    # evaluation); a value on an E4M3 rounding boundary then takes the
    # neighbouring code, one E4M3 step (up to 2^-3 of the element) away. The
    # down-projection is therefore checked to the bf16 bound against the
    # oracle's own FP8 down-projection of the GPU's H, and end to end against
    # a bound for such steps: one step in one of the f terms of a row moves it
    # by up to about 0.5 / sqrt(f) of max|O| (fp8_fwd_tol).
    o_tol = {}
    if w.fp8:
        check_fp8_down_own_h(w, L, f, off, rep)
        if w.fp8_scale in ("block", "square"):
            check_fp8_h_codes(w, L, dev, off)
        o_tol = fp8_fwd_tol(w.f)
    assert_close("O", to_np(L.out[:A])[g_rows], fwd["O"][o_rows], dt, rep, **o_tol)
    if w.n_shared:
        assert_close("O_shared", to_np(L.out_shared), fwd["Os"], dt, rep, **o_tol)
    assert_close("Y", to_np(L.Y)[tok_ok], fwd["Y"][tok_ok], dt, rep, **o_tol)
    # ---- backward
    if w.fp8:
        # dgate = <dY, O> of the GPU's own O, to the bf16 bound; downstream of O
        # (dgate, the router gradients, dX through dx_router) the end-to-end
        # comparison takes O's bound
        rowg = L.row_of.cpu().numpy().astype(np.int64)
        own = np.zeros(rowg.shape)
        if A:
            Og = to_np(L.out[:A])
            own = np.einsum("tc,tjc->tj", f["dy"], Og[np.maximum(rowg, 0)])
            own = np.where(rowg >= 0, own, 0.0)
        assert_close("dgate(own O)", to_np(L.dgate), own, dt, rep)
    assert_close("dgate", to_np(L.dgate)[tok_ok], bwd["dgate"][tok_ok], dt, rep, **o_tol)
    # gradients of a row also carry its token's gate: skip rows of flipped tokens
    keep = tok_ok[token_of[g_rows]] if len(g_rows) else np.zeros(0, bool)
    assert_close("dO", to_np(L.dout[:A])[g_rows[keep]], bwd["dO"][o_rows[keep]], dt, rep)
    # outputs computed from a requantized operand (FP8 data gradients) carry
    # the matrix core's accumulation error amplified by E4M3 rounding: see
    # check_fp8_dgrad for the exact checks and fp8_dgrad_tol for this bound
    dxt = fp8_dgrad_tol(w.f, w.fp8_grad) if w.fp8_bwd else {}
    assert_close("dX_perm", to_np(L.dx_perm[:A])[g_rows[keep]], bwd["dx_perm"][o_rows[keep]], dt, rep,
                 **dxt)
    gw13, gw2 = to_np(L.dw13), to_np(L.dw2)
    # FP8 weight gradients: see fp8_wgrad_tol (exact stage check in check_fp8_wgrad)
    rows = np.diff(off)
    wgt = fp8_wgrad_tol(int(rows[rows > 0].min(initial=w.T)), w.fp8_grad) if w.fp8_wgrad else {}
    assert_close("dW13", gw13[e_ok], bwd["dw13"][e_ok], dt, rep, **wgt)
    assert_close("dW2", gw2[e_ok], bwd["dw2"][e_ok], dt, rep, **wgt)
    empty = [e for e in range(E) if off[e + 1] == off[e]]
    for e in empty:   # an expert without rows has exactly zero gradient
        assert not gw13[e].any() and not gw2[e].any()
    if w.n_shared:
        assert_close("dX_shared", to_np(L.dx_shared), bwd["dx_shared"], dt, rep, **dxt)
        swt = fp8_wgrad_tol(w.T, w.fp8_grad) if w.fp8_wgrad else {}
        assert_close("dSW13", to_np(L.dsw13), bwd["dsw13"], dt, rep, **swt)
        assert_close("dSW2", to_np(L.dsw2), bwd["dsw2"], dt, rep, **swt)
    # The router gradient can vanish identically (top-1: the one renormalised
    # gate is constant 1), leaving only fp32 rounding of g (1 - g) dg on the
    # GPU; an absolute floor scaled by the formula's inputs covers that case.
    dl_floor = 2e-6 * float(np.abs(bwd["dgate"]).max(initial=0.0))
    assert_close("dlogits", to_np(L.dlogits)[tok_ok], bwd["dlogits"][tok_ok], dt, rep,
                 atol=dl_floor, **o_tol)
    # router weight gradient: against the oracle, and exactly dl^T x of the
    # GPU's own dl (a property of the definition that holds at any size)
    gdl = to_np(L.dlogits)
    assert_close("dW_r(own dl)", to_np(L.dw_r), gdl.T @ f["x"], dt, rep, rel=2e-5)
    assert_close("dx_router(own dl)", to_np(L.dx_router), gdl @ f["w_r"], dt, rep, rel=2e-5)
    if not bad_e:
        assert_close("dW_r", to_np(L.dw_r), bwd["dw_r"], dt, rep,
                     atol=dl_floor * float(np.abs(f["x"]).sum(axis=0).max(initial=0.0)), **o_tol)
    dxo = dict(dxt)
    if o_tol:
        dxo["max_rel"] = max(dxo.get("max_rel", 2e-2), o_tol["max_rel"])
    assert_close("dX", to_np(L.dX)[tok_ok], bwd["dX"][tok_ok], dt, rep, **dxo)
    if w.fp8_bwd:
        check_fp8_dgrad(w, L, dev, bwd, rep, g_rows[keep], o_rows[keep], off)
    if w.fp8_wgrad:
        check_fp8_wgrad(w, L, dev, rep, off)
    return len(flips)


# FP8 bounds where each side quantizes a bf16 tensor it computed itself (H in
# the forward, dpre in the data gradients). float32 on the device against
# float64 in the oracle moves some bf16 values by one bf16 step, and a value
# at an E4M3 rounding boundary then takes the neighbouring code, one E4M3 step
# (2^-4 to 2^-3 of the element) away. One such code moves an output element
# by up to about 0.42 / sqrt(f) of the tensor's max (derived, and measured on
# an emulation of the device arithmetic, in tests/test_fp8_tolerance.py).
# The exact stage checks (check_fp8_down_own_h, check_fp8_dgrad) hold each
# FP8 product of the GPU's own bf16 operand to the bf16 bound.
def fp8_fwd_tol(f):
    return dict(max_rel=max(2e-2, 0.5 / np.sqrt(f)))


def fp8_dgrad_tol(f, fmt="e4m3"):
    """E5M2 gradient operands: one E5M2 step is up to 2^-2 of its element,
    twice E4M3's, so the bound doubles."""
    if fmt == "e5m2":
        return dict(max_rel=max(1e-1, 1.0 / np.sqrt(f)), l1_rel=3e-2)
    return dict(max_rel=max(5e-2, 0.5 / np.sqrt(f)), l1_rel=1.5e-2)


# FP8 weight gradients: a weight-gradient element sums n tokens' products, and
# a token whose bf16 operand (dO, H or dpre) the two sides round differently at
# an E4M3 boundary moves one term by one E4M3 step (up to 2^-3 of it); against
# max|dW| of about 4 sqrt(n) rms(a) rms(b) that is up to about 0.5 / sqrt(n)
# for the smallest expert's n tokens. dpre also carries the FP8 data gradient's
# bound. The stage check (check_fp8_wgrad) holds each weight gradient of the
# GPU's own bf16 operands to the bf16 bound.
def fp8_wgrad_tol(n, fmt="e4m3"):
    if fmt == "e5m2":
        return dict(max_rel=max(1e-1, 1.0 / np.sqrt(max(n, 1))), l1_rel=3e-2)
    return dict(max_rel=max(5e-2, 0.5 / np.sqrt(max(n, 1))), l1_rel=1.5e-2)


def check_fp8_wgrad(w, L, dev, rep, off):
    """The FP8 weight gradients of the GPU's own bf16 operands (dO, H, dpre,
    x_perm; for the shared expert dY, its H and dpre and x), recomputed by the
    oracle's expert_wgrad_fp8, to the bf16 bound. The layer's later calls
    reuse the workspace, so the backward is rerun into a fresh one (it is
    deterministic: check_fp8_dgrad compares the rerun with the layer bitwise)
    and dpre is read from there."""
    import mixture_experts_layer_28_amd as moe
    A = int(off[-1])
    R, P = w.T * w.k, (2 * w.f if w.act == "swiglu" else w.f)
    ws = torch.empty_like(L.ws)
    like = lambda t: torch.empty_like(t) if t is not None else None   # noqa: E731
    o = {n: like(getattr(L, n)) for n in ("dx_perm", "dx_shared", "dw13", "dw2", "dsw13", "dsw2")}
    moe.grouped_ffn_bwd_fp8(L.desc, L.x_perm, L.offsets, dev["x"], L.w13q_t, L.s13_t, L.w2q_t,
                            L.s2_t, L.sw13q_t, L.ss13_t, L.sw2q_t, L.ss2_t, L.save_pre, L.save_h,
                            L.save_pre_s, L.save_h_s, L.dout, dev["dy"], o["dx_perm"],
                            o["dx_shared"], o["dw13"], o["dw2"], o["dsw13"], o["dsw2"], ws,
                            fp8_wgrad=True, block=w.fp8_scale == "square")
    torch.cuda.synchronize()
    assert torch.equal(o["dw13"], L.dw13) and torch.equal(o["dw2"], L.dw2)
    dO, H, X = (to_np(t[:A]) for t in (L.dout, L.save_h, L.x_perm))
    dp = to_np(ws[: R * P * 2].view(torch.bfloat16).view(R, P)[:A])
    for e in range(w.E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        g13, g2 = O.expert_wgrad_fp8(X[r0:r1], H[r0:r1], dO[r0:r1], dp[r0:r1], w.fp8_grad)
        assert_close(f"dW13(own) e{e}", to_np(L.dw13[e]), g13, "bf16", rep)
        assert_close(f"dW2(own) e{e}", to_np(L.dw2[e]), g2, "bf16", rep)
    if w.n_shared:
        off_s = (R * P * 2 + 255) // 256 * 256
        dps = to_np(ws[off_s: off_s + w.T * P * 2].view(torch.bfloat16).view(w.T, P))
        g13, g2 = O.expert_wgrad_fp8(to_np(dev["x"]), to_np(L.save_h_s), to_np(dev["dy"]), dps,
                                     w.fp8_grad)
        assert_close("dSW13(own)", to_np(L.dsw13[0]), g13, "bf16", rep)
        assert_close("dSW2(own)", to_np(L.dsw2[0]), g2, "bf16", rep)


def _fp8_rows_ref(M, fmt="e4m3"):
    """_e4m3_rows_ref for either FP8 format: the scale by search around
    log2(amax / M_fmt), the codes by torch's float8_e4m3fn or float8_e5m2 cast."""
    if fmt == "e4m3":
        return _e4m3_rows_ref(M)
    M = np.asarray(M, dtype=np.float64)
    amax = np.abs(M).max(axis=1, initial=0.0)
    safe = np.where(amax > 0, amax, 57344.0)
    e = np.floor(np.log2(safe / 57344.0)).astype(np.int64) - 1
    for _ in range(3):
        e = np.where(amax > 57344.0 * np.exp2(e.astype(np.float64)), e + 1, e)
    e = np.where(amax > 0, e, 0)
    sc = np.exp2(e.astype(np.float64))[:, None]
    q = torch.from_numpy(M / sc).to(torch.float32).to(torch.float8_e5m2).to(torch.float64)
    return q.numpy() * sc


def check_grad_codes(w, L, dev, ws, R, P, A, dp, dps):
    """The FP8 backward's codes and scales of its gradient operands (the
    upstream gradient and dpre), read from the workspace it left, against the
    oracle's quantizer in the chosen format on the same bf16 rows: per-row
    exponents, or (square mode) the block-scale bytes of 32-element blocks."""
    import mixture_experts_layer_28_amd as moe
    d = w.d
    blk = w.fp8_scale == "square"
    al = lambda x: (x + 255) // 256 * 256   # noqa: E731
    base = moe.workspace_size(L.desc, moe.MOE_OP_FFN_BWD)
    raw = ws.cpu().numpy()
    if dps is not None:
        rows, g_src, p_src = w.T, to_np(dev["dy"]), dps
    else:
        rows, g_src, p_src = A, to_np(L.dout[:A]), dp
    gsb = moe.fp8_block_scale_bytes(R, d) if blk else 4 * R
    psb = moe.fp8_block_scale_bytes(R, P) if blk else 4 * R
    gq = raw[base: base + R * d].reshape(R, d)[:rows]
    gs = raw[base + al(R * d): base + al(R * d) + gsb]
    o_pq = base + al(R * d) + al(gsb)
    pq = raw[o_pq: o_pq + R * P].reshape(R, P)[:rows]
    ps = raw[o_pq + al(R * P): o_pq + al(R * P) + psb]
    for name, q, sbuf, src, K in (("dO", gq, gs, g_src, d), ("dpre", pq, ps, p_src, P)):
        if blk:
            rc, re_ = O.quantize_blocks_fp8(src, fmt=w.fp8_grad)
            got_e = block_bytes(sbuf, rows, K)[:, : re_.shape[1]].astype(np.int64) - 127
        else:
            rc, re_ = O.quantize_rows_fp8(src, w.fp8_grad)
            got_e = sbuf.view(np.int32)[:rows]
        assert (got_e == re_).all(), f"{name} exponents differ ({w.fp8_grad})"
        bad = np.argwhere(q != rc)
        assert bad.size == 0, f"{name} {w.fp8_grad} codes differ: {len(bad)}, first {bad[:4].tolist()}"


def _e4m3_rows_ref(M):
    """Dequantized per-row E4M3 of M (rows of bf16 values) by an independent
    route: the scale exponent by a search around log2(amax/448), the codes by
    torch's float8_e4m3fn cast."""
    M = np.asarray(M, dtype=np.float64)
    amax = np.abs(M).max(axis=1, initial=0.0)
    safe = np.where(amax > 0, amax, 448.0)
    e = np.floor(np.log2(safe / 448.0)).astype(np.int64) - 1
    for _ in range(3):                       # smallest e with amax <= 448 * 2^e
        e = np.where(amax > 448.0 * np.exp2(e.astype(np.float64)), e + 1, e)
    e = np.where(amax > 0, e, 0)
    sc = np.exp2(e.astype(np.float64))[:, None]
    q = torch.from_numpy(M / sc).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64)
    return q.numpy() * sc


def _decode_codes(codes, sexp):
    """Dequantized rows of device E4M3 codes [n, K] with exponents [n]."""
    v = codes.cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return v * np.exp2(sexp.cpu().numpy().astype(np.float64))[:, None]


def check_fp8_dgrad(w, L, dev, bwd, rep, g_rows, o_rows, off):
    """The FP8 backward stage by stage: rerun it on the layer's saved tensors
    into fresh buffers (bitwise identical: deterministic); read its bf16
    pre-activation gradient dpre from the workspace and compare it with the
    oracle's; and check dX against the FP8 product of the GPU's own dpre,
    requantized by _e4m3_rows_ref (square mode: the oracle's 32-element
    blocks), with the GPU's transposed weight codes."""
    import mixture_experts_layer_28_amd as moe
    dt = w.dtype
    A = int(off[-1])
    R, P = w.T * w.k, (2 * w.f if w.act == "swiglu" else w.f)
    ws = torch.empty_like(L.ws)
    like = lambda t: torch.empty_like(t) if t is not None else None   # noqa: E731
    o = {n: like(getattr(L, n)) for n in ("dx_perm", "dx_shared", "dw13", "dw2", "dsw13", "dsw2")}
    moe.grouped_ffn_bwd_fp8(L.desc, L.x_perm, L.offsets, dev["x"], L.w13q_t, L.s13_t, L.w2q_t,
                            L.s2_t, L.sw13q_t, L.ss13_t, L.sw2q_t, L.ss2_t, L.save_pre, L.save_h,
                            L.save_pre_s, L.save_h_s, L.dout, dev["dy"], o["dx_perm"],
                            o["dx_shared"], o["dw13"], o["dw2"], o["dsw13"], o["dsw2"], ws,
                            fp8_wgrad=w.fp8_wgrad, block=w.fp8_scale == "square")
    torch.cuda.synchronize()
    assert torch.equal(o["dx_perm"][:A], L.dx_perm[:A]), "FP8 backward is not deterministic"
    assert torch.equal(o["dw13"], L.dw13) and torch.equal(o["dw2"], L.dw2)
    dpre = ws[: R * P * 2].view(torch.bfloat16).view(R, P)
    assert_close("dpre", to_np(dpre[:A])[g_rows], bwd["dpre"][o_rows], dt, rep)
    sq = w.fp8_scale == "square"
    if sq:
        w13t = decode_block_codes(L.w13q_t.reshape(w.E * w.d, P), L.s13_t).reshape(w.E, w.d, P)

        def qg(m):
            return O.dequantize_blocks_fp8(*O.quantize_blocks_fp8(m, fmt=w.fp8_grad), fmt=w.fp8_grad)
    else:
        w13t = [_decode_codes(L.w13q_t[e], L.s13_t[e]) for e in range(w.E)]   # [d, P] each

        def qg(m):
            return _fp8_rows_ref(m, w.fp8_grad)
    dp = to_np(dpre[:A])
    got, ref = [], []
    for e in range(w.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            ref.append(qg(dp[lo:hi]) @ w13t[e].T)
            got.append(to_np(L.dx_perm[lo:hi]))
    if got:
        assert_close("dX_perm(own dpre)", np.concatenate(got), np.concatenate(ref), dt, rep)
    if w.n_shared:
        off_s = (R * P * 2 + 255) // 256 * 256
        dps = to_np(ws[off_s: off_s + w.T * P * 2].view(torch.bfloat16).view(w.T, P))
        assert_close("dpre_shared", dps, bwd["dpre_shared"], dt, rep)
        wst = decode_block_codes(L.sw13q_t[0], L.ss13_t) if sq else _decode_codes(L.sw13q_t[0], L.ss13_t[0])
        assert_close("dX_shared(own dpre)", to_np(L.dx_shared), qg(dps) @ wst.T, dt, rep)
    # the gradient codes in the workspace, bit for bit (E4M3 or E5M2): the
    # shared expert's rows overwrite the routed ones when there is one
    check_grad_codes(w, L, dev, ws, R, P, A, dp, dps if w.n_shared else None)


def check_fp8_h_codes(w, L, dev, off):
    """The block-scaled forward writes H's FP8 codes and block-scale bytes in
    its up-projection's epilogue: rerun the forward into fresh buffers (it is
    deterministic: the rerun's H and O equal the layer's bitwise) and compare
    the codes and exponents it leaves in the workspace with the oracle's
    block quantizer on the same bf16 H, bit for bit (routed rows, and the
    shared expert's)."""
    import mixture_experts_layer_28_amd as moe
    A, R, f = int(off[-1]), w.T * w.k, w.f
    al = lambda x: (x + 255) // 256 * 256   # noqa: E731
    ws = torch.empty_like(L.ws)
    like = lambda t: torch.empty_like(t) if t is not None else None   # noqa: E731
    o = {n: like(getattr(L, n)) for n in ("save_pre", "save_h", "save_pre_s", "save_h_s", "out", "out_shared")}
    moe.grouped_ffn_fwd_fp8b(L.desc, L.xq_perm, L.sx_perm, L.offsets, L.xq, L.sx, L.w13q, L.s13, L.w2q, L.s2,
                             L.sw13q, L.ss13, L.sw2q, L.ss2, o["save_pre"], o["save_h"], o["save_pre_s"],
                             o["save_h_s"], o["out"], o["out_shared"], ws)
    torch.cuda.synchronize()
    assert torch.equal(o["save_h"][:A], L.save_h[:A]) and torch.equal(o["out"][:A], L.out[:A])
    raw = ws.cpu().numpy()
    SB = moe.fp8_block_scale_bytes(R, f)
    parts = [(A, 0, al(R * f), to_np(L.save_h[:A]))]
    if w.n_shared:
        base = al(R * f) + al(SB)
        parts.append((w.T, base, base + al(w.T * f), to_np(L.save_h_s)))
    for rows, c0, s0, H in parts:
        if rows == 0:
            continue
        codes = raw[c0: c0 + rows * f].reshape(rows, f)
        rc, re_ = O.quantize_blocks_fp8(H)
        bad = np.argwhere(codes != rc)
        assert bad.size == 0, f"H codes differ: {len(bad)}, first {bad[:4].tolist()}"
        got = block_bytes(raw[s0:], rows, f).astype(np.int64)
        nb = re_.shape[1]
        assert (got[:, :nb] - 127 == re_).all(), "H block exponents differ"
        assert (got[:, nb:] == 127).all(), "H padding blocks are not 127"


def check_fp8_down_own_h(w, L, f, off, rep):
    """FP8 down-projection of the GPU's own bf16 H (routed experts, and the
    shared expert on all tokens), recomputed by the oracle: E4M3 codes of H
    against the quantized W2 (per row, per 32-element block with fp8_scale
    "block", 32 x 32 squares with "square"), held to the bf16 bound."""
    if w.fp8_scale in ("block", "square"):
        qa = lambda m: O.dequantize_blocks_fp8(*O.quantize_blocks_fp8(m))   # noqa: E731
        qw = O.quantize_weights_fp8_square if w.fp8_scale == "square" else O.quantize_weights_fp8_block
    else:
        qa = lambda m: O.dequantize_rows_fp8(*O.quantize_rows_fp8(m))   # noqa: E731
        qw = O.quantize_weights_fp8
    A = int(off[-1])
    Hg = to_np(L.save_h[:A]).astype(np.float64)
    Og = to_np(L.out[:A]).astype(np.float64)
    w2 = f["w2"]
    for e in range(w.E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        own = qa(Hg[r0:r1]) @ qw(w2[e]).T
        assert_close(f"O(own H) e{e}", Og[r0:r1], own, "bf16", rep)
    if w.n_shared:
        hs = to_np(L.save_h_s).astype(np.float64)
        sw2 = f["sw2"][0]
        own = qa(hs) @ qw(sw2).T
        assert_close("O_shared(own H)", to_np(L.out_shared).astype(np.float64), own, "bf16", rep)


def run_and_compare(w: Workload, g=None):
    g = g if g is not None else gen_all(w)
    L, dev = gpu_layer(w, g)
    fwd, bwd, f = oracle_layer(w, g)
    rep = Report()
    flips = compare_layer(w, L, dev, fwd, bwd, f, rep)
    return rep, flips, L, dev
