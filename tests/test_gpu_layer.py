"""GPU parity of the whole layer (forward + backward) against the CPU oracle,
stage by stage, at sizes the oracle finishes in seconds but that still span
several tiles with ragged tails; plus edge cases and determinism."""
import numpy as np
import pytest
import torch

from moe_inputs import WORKLOADS, Workload, gen_all
from parity_util import bits, run_and_compare, to_dev, to_np

pytestmark = pytest.mark.gpu

REDUCED = {
    # the tiny fp32 workload at its full size
    "tiny_fp32": WORKLOADS["tiny_fp32"],
    # the four bf16 workloads with their structure (E, k, scoring, FFN, bias,
    # capacity, shared expert) at reduced T, d, f
    "mixtral_small": WORKLOADS["mixtral_bf16"].replace(T=1536, d=512, f=768),
    "skewed_cf1_small": WORKLOADS["skewed_bf16"].replace(T=1024, d=512, f=1024),
    "skewed_nocap_small": WORKLOADS["skewed_nocap_bf16"].replace(T=1024, d=512, f=1024),
    "finegrained_small": WORKLOADS["finegrained_bf16"].replace(T=2048, d=512, f=256),
    "dsv3_small": WORKLOADS["dsv3_bf16"].replace(T=1024, d=512, f=256),
    # the noisy (Gumbel) gate on the Mixtral-like structure, with aux and z-loss terms
    "mixtral_noisy_small": WORKLOADS["mixtral_noisy_bf16"].replace(T=1536, d=512, f=768),
    # top-1 routing and a 1.5 capacity factor on the skewed load
    "top1_small": WORKLOADS["top1_bf16"].replace(T=1536, d=512, f=768),
    "skewed_cf15_small": WORKLOADS["skewed_cf15_bf16"].replace(T=1024, d=512, f=1024),
    # FP8 forward GEMMs (routed only; routed + shared with sigmoid scoring)
    "mixtral_fp8_small": WORKLOADS["mixtral_fp8_bf16"].replace(T=1536, d=512, f=768),
    "dsv3_fp8_small": WORKLOADS["dsv3_bf16"].replace(T=1024, d=512, f=256, fp8=True),
    # FP8 forward GEMMs with one scale per 32 elements along K
    "mixtral_fp8b_small": WORKLOADS["mixtral_fp8b_bf16"].replace(T=1536, d=512, f=768),
    "dsv3_fp8b_small": WORKLOADS["dsv3_bf16"].replace(T=1024, d=512, f=256, fp8=True,
                                                      fp8_scale="block"),
    # every GEMM on FP8 operands (weight gradients: token-axis block scales)
    "mixtral_fp8_all_small": WORKLOADS["mixtral_fp8_all_bf16"].replace(T=1536, d=512, f=768),
    "dsv3_fp8_all_small": WORKLOADS["dsv3_bf16"].replace(T=1024, d=512, f=256, fp8=True,
                                                         fp8_bwd=True, fp8_wgrad=True),
    # and with E5M2 gradient operands (dO, dpre)
    "mixtral_fp8_all_e5m2_small": WORKLOADS["mixtral_fp8_all_e5m2_bf16"].replace(T=1536, d=512,
                                                                                f=768),
    "dsv3_fp8_all_e5m2_small": WORKLOADS["dsv3_bf16"].replace(T=1024, d=512, f=256, fp8=True,
                                                              fp8_bwd=True, fp8_wgrad=True,
                                                              fp8_grad="e5m2"),
    # FP8 forward and FP8 data gradients (weight gradients bf16)
    "mixtral_fp8_dgrad_small": WORKLOADS["mixtral_fp8_dgrad_bf16"].replace(T=1536, d=512, f=768),
    "dsv3_fp8_dgrad_small": WORKLOADS["dsv3_bf16"].replace(T=1024, d=512, f=256, fp8=True,
                                                           fp8_bwd=True),
    # square-block weights: forward and data gradients on block scales (and the
    # weight gradients on token-axis blocks; E5M2 gradient operands)
    "mixtral_fp8sq_dgrad_small": WORKLOADS["mixtral_fp8sq_dgrad_bf16"].replace(T=1536, d=512, f=768),
    "dsv3_fp8sq_all_small": WORKLOADS["dsv3_bf16"].replace(T=1024, d=512, f=256, fp8=True,
                                                           fp8_bwd=True, fp8_wgrad=True,
                                                           fp8_scale="square"),
    "mixtral_fp8sq_all_e5m2_small": WORKLOADS["mixtral_fp8sq_all_bf16"].replace(T=1536, d=512, f=768,
                                                                               fp8_grad="e5m2"),
}

EDGE = {
    # ragged everything: T, E, d (K tail of 8), f (N tails), k=3, shared GELU, sigmoid
    "ragged_gelu_shared": Workload("ragged", T=1000, d=136, E=6, k=3, f=200, act="gelu",
                                   score="sigmoid", n_shared=1, sel_bias=True, aux_coef=0.1,
                                   bias_gamma=0.01),
    "ragged_swiglu_fp32": Workload("ragged32", T=333, d=72, E=5, k=2, f=40, dtype="fp32",
                                   cf=0.8, aux_coef=0.05, z_coef=0.05),
    # capacity 0: every assignment dropped, only the shared expert remains
    "all_dropped_shared": Workload("drop", T=512, d=256, E=8, k=2, f=256, cf=0.0, n_shared=1),
    # all tokens on one expert (logit bias), top-1, capacity keeps the first C
    "one_hot_expert": Workload("onehot", T=700, d=256, E=4, k=1, f=256, cf=1.0,
                               logit_bias={2: 50.0}),
    # one expert, top-1: a dense FFN
    "single_expert": Workload("single", T=300, d=128, E=1, k=1, f=384),
    # E at the router's 1024-expert limit region and k at 16
    "wide_router": Workload("wide", T=256, d=64, E=320, k=16, f=64, aux_coef=0.02, z_coef=0.01),
    # the library's limit of 1024 experts: the grouped GEMMs' group prefix
    # covers all 1024 groups (most hold 0-4 rows), router and statistics at E = 1024
    "max_experts": Workload("e1024", T=640, d=64, E=1024, k=4, f=64, aux_coef=0.01),
    # noisy gate through the GEMM-logits router (E > 8), fp32, low temperature
    "noisy_fp32": Workload("noisy32", T=300, d=64, E=40, k=4, f=64, dtype="fp32", gumbel_tau=0.5,
                           aux_coef=0.05, z_coef=0.02),
    # router logits split over K (few T x E tiles, d >= 512) with a logit bias in
    # partition 0, E = 40 (an N tail of the 64-wide tile), dense dl from the
    # aux and z losses; then float32 with d = 1032 (a K tail of 8 in the last
    # partition) and E = 20 (dl's rows not 8-aligned: dW_r and dx on the ALU)
    "router_splitk_bias": Workload("rsplit", T=777, d=1024, E=40, k=4, f=64,
                                   logit_bias={3: 1.5, 17: -2.0}, aux_coef=0.02, z_coef=0.01),
    "router_splitk_ktail_fp32": Workload("rsplit32", T=515, d=1032, E=20, k=2, f=48,
                                         dtype="fp32", logit_bias={0: 1.0}, aux_coef=0.05),
    # bf16 router products on the bf16 matrix cores (E a multiple of 8): d = 1032
    # and T = 515 leave one partition each with a K tail (8 columns of x, 3
    # tokens), dense dl from the aux and z losses, a logit bias in the fold
    "router_bf16_split_ktail": Workload("rx3tail", T=515, d=1032, E=24, k=3, f=64,
                                        logit_bias={5: 1.25, 20: -0.75}, aux_coef=0.05,
                                        z_coef=0.02),
    # FP8 forward with ragged T, E, a K tail (d = 144 = 2*64 + 16) and N tails
    # (f = 208), GELU and a shared expert
    "ragged_fp8_gelu_shared": Workload("ragged8", T=1000, d=144, E=6, k=3, f=208, act="gelu",
                                       score="sigmoid", n_shared=1, sel_bias=True, fp8=True),
    # whole five-k-step ring trips and no tail: d = 320 and f = 640 give the bf16
    # GEMMs 5 and 10 k-steps of 64 (the FP8 ones 3 and 5 of 128)
    "ring_whole_trips": Workload("ring5", T=700, d=320, E=4, k=2, f=640, aux_coef=0.02),
    "ring_whole_trips_fp8": Workload("ring5f8", T=700, d=320, E=4, k=2, f=640, fp8=True),
    # FP8 forward with every assignment dropped: the routed GEMMs see no rows
    "fp8_all_dropped_shared": Workload("drop8", T=512, d=256, E=8, k=2, f=256, cf=0.0,
                                       n_shared=1, fp8=True),
    # FP8 data gradients: ragged sizes with GELU and a shared expert; whole
    # ring trips (dX: K = 2f = 1280, ten 128-k steps); every assignment
    # dropped; and FP8 data gradients after a bf16 forward
    "ragged_fp8_dgrad_gelu_shared": Workload("ragged8d", T=1000, d=144, E=6, k=3, f=208,
                                             act="gelu", score="sigmoid", n_shared=1,
                                             sel_bias=True, fp8=True, fp8_bwd=True),
    "ring_whole_trips_fp8_dgrad": Workload("ring5f8d", T=700, d=320, E=4, k=2, f=640, fp8=True,
                                           fp8_bwd=True),
    "fp8_dgrad_all_dropped_shared": Workload("drop8d", T=512, d=256, E=8, k=2, f=256, cf=0.0,
                                             n_shared=1, fp8=True, fp8_bwd=True),
    "fp8_dgrad_only": Workload("dg8", T=600, d=256, E=4, k=2, f=384, aux_coef=0.02,
                               fp8_bwd=True),
    # block-scaled FP8 forward: K tails with a partial last block and padding
    # bytes (d = 144: blocks 0-4, the last of 16; f = 208: blocks 0-6, the last
    # of 16), whole ring trips, no routed rows, and FP8 data gradients after it
    "ragged_fp8b_gelu_shared": Workload("ragged8b", T=1000, d=144, E=6, k=3, f=208, act="gelu",
                                        score="sigmoid", n_shared=1, sel_bias=True, fp8=True,
                                        fp8_scale="block"),
    "ring_whole_trips_fp8b": Workload("ring5f8b", T=700, d=320, E=4, k=2, f=640, fp8=True,
                                      fp8_scale="block"),
    "fp8b_all_dropped_shared": Workload("drop8b", T=512, d=256, E=8, k=2, f=256, cf=0.0,
                                        n_shared=1, fp8=True, fp8_scale="block"),
    "fp8b_fwd_fp8_dgrad": Workload("f8bd", T=600, d=256, E=4, k=2, f=384, fp8=True,
                                   fp8_bwd=True, fp8_scale="block"),
    # FP8 weight gradients: ragged experts (rows off every 32- and 128-token
    # step), K tails, GELU and a shared expert; no routed rows; every token on
    # one expert (the others empty); and after the block-scaled forward
    "ragged_fp8_all_gelu_shared": Workload("ragged8w", T=1000, d=144, E=6, k=3, f=208,
                                           act="gelu", score="sigmoid", n_shared=1,
                                           sel_bias=True, fp8=True, fp8_bwd=True,
                                           fp8_wgrad=True),
    "fp8_all_dropped_shared": Workload("drop8w", T=512, d=256, E=8, k=2, f=256, cf=0.0,
                                       n_shared=1, fp8=True, fp8_bwd=True, fp8_wgrad=True),
    "fp8_all_one_expert": Workload("onehot8w", T=700, d=256, E=4, k=1, f=256,
                                   logit_bias={2: 50.0}, fp8=True, fp8_bwd=True, fp8_wgrad=True),
    "fp8b_fwd_fp8_all": Workload("f8bw", T=600, d=256, E=4, k=2, f=384, fp8=True, fp8_bwd=True,
                                 fp8_wgrad=True, fp8_scale="block"),
    # E5M2 gradient operands: ragged sizes with GELU and a shared expert, and
    # E5M2 data gradients with bf16 weight gradients after a bf16 forward
    "ragged_fp8_all_e5m2_gelu_shared": Workload("ragged8e5", T=1000, d=144, E=6, k=3, f=208,
                                                act="gelu", score="sigmoid", n_shared=1,
                                                sel_bias=True, fp8=True, fp8_bwd=True,
                                                fp8_wgrad=True, fp8_grad="e5m2"),
    "fp8_e5m2_dgrad_only": Workload("dg8e5", T=600, d=256, E=4, k=2, f=384, aux_coef=0.02,
                                    fp8_bwd=True, fp8_grad="e5m2"),
    # the 1024-expert limit with every FP8 mode at once (block-scaled forward,
    # FP8 data and weight gradients: a 1024-group k-step table), and one token
    "max_experts_fp8_all": Workload("e1024f8", T=640, d=64, E=1024, k=4, f=64, aux_coef=0.01,
                                    fp8=True, fp8_bwd=True, fp8_wgrad=True, fp8_scale="block"),
    "one_token_fp8_all": Workload("t1f8", T=1, d=128, E=4, k=2, f=96, n_shared=1, fp8=True,
                                  fp8_bwd=True, fp8_wgrad=True, fp8_grad="e5m2"),
    # square-block weights: partial squares at both edges (d 144, f 208) with
    # GELU and a shared expert; no routed rows; square data gradients after a
    # bf16 forward (the backward quantizes the transposes only), E5M2; the
    # square forward alone (rows only); 1024 experts
    "ragged_fp8sq_gelu_shared": Workload("ragged8sq", T=1000, d=144, E=6, k=3, f=208, act="gelu",
                                         score="sigmoid", n_shared=1, sel_bias=True, fp8=True,
                                         fp8_bwd=True, fp8_scale="square"),
    "fp8sq_all_dropped_shared": Workload("drop8sq", T=512, d=256, E=8, k=2, f=256, cf=0.0,
                                         n_shared=1, fp8=True, fp8_bwd=True, fp8_wgrad=True,
                                         fp8_scale="square"),
    "fp8sq_e5m2_dgrad_only": Workload("dg8sq", T=600, d=256, E=4, k=2, f=384, aux_coef=0.02,
                                      fp8_bwd=True, fp8_scale="square", fp8_grad="e5m2"),
    "fp8sq_fwd_only": Workload("fw8sq", T=600, d=256, E=4, k=2, f=384, n_shared=1, fp8=True,
                               fp8_scale="square"),
    "max_experts_fp8sq_all": Workload("e1024sq", T=640, d=64, E=1024, k=4, f=64, aux_coef=0.01,
                                      fp8=True, fp8_bwd=True, fp8_wgrad=True, fp8_scale="square"),
}


@pytest.mark.parametrize("name", list(REDUCED))
def test_layer_parity(name):
    w = REDUCED[name]
    print(f"[case] {name} {w}", flush=True)
    rep, flips, L, dev = run_and_compare(w)
    print(rep, flush=True)


@pytest.mark.parametrize("name", list(EDGE))
def test_layer_edge_cases(name):
    w = EDGE[name]
    print(f"[case] {name} {w}", flush=True)
    rep, flips, L, dev = run_and_compare(w)
    print(rep, flush=True)
    if name == "all_dropped_shared":
        assert int(L.offsets[-1]) == 0
        assert not to_np(L.dw13).any() and not to_np(L.dw2).any()
    if name == "one_hot_expert":
        off = L.offsets.cpu().numpy()
        assert list(np.diff(off)) == [0, 0, 175, 0]
        assert (L.token_of[:175].cpu().numpy() == np.arange(175)).all()


def test_fp8_block_scales_follow_the_blocks():
    """Inputs whose 32-column blocks span many binades: x's blocks scaled by
    2^s_b, s_b in [-10, 10], with the matching input columns of w13 and of
    the router weight scaled by 2^-s_b (products and router logits are
    unchanged), and w2's blocks by 2^r_b, r_b in [-4, 4]. Each block's scale
    then differs from its neighbours', so a scale applied to the wrong block,
    or one scale per row, misses the oracle's block-scaled result by far more
    than the FP8 bound (test_fp8_tolerance.py shows both on the CPU)."""
    from moe_inputs import bf16_bits_to_f32, to_bf16_bits
    w = WORKLOADS["mixtral_fp8b_bf16"].replace(T=768, d=384, f=512, seed=5)
    print(f"[case] fp8 block scales {w}", flush=True)
    g = gen_all(w)
    rng = np.random.default_rng(11)
    sx = np.exp2(rng.integers(-10, 11, w.d // 32)).astype(np.float32)
    sw = np.exp2(rng.integers(-4, 5, w.f // 32)).astype(np.float32)
    col = lambda s: np.repeat(s, 32)   # noqa: E731
    g["x"] = to_bf16_bits(bf16_bits_to_f32(g["x"]) * col(sx))
    g["w13"] = to_bf16_bits(bf16_bits_to_f32(g["w13"]) / col(sx))
    g["w_r"] = (g["w_r"] / col(sx)).astype(np.float32)
    g["w2"] = to_bf16_bits(bf16_bits_to_f32(g["w2"]) * col(sw))
    rep, flips, L, dev = run_and_compare(w, g)
    print(rep, flush=True)


def test_fp8_square_scales_follow_the_squares():
    """Weights whose 32 x 32 squares span many binades: each square of w13
    and w2 scaled by its own 2^s, s in [-5, 5]. A square's byte applied to
    another square (a transposed or shifted scale array, the forward's row
    layout read as the transpose's) then misses the oracle's square-scaled
    forward and data gradients by far more than the FP8 bound."""
    from moe_inputs import bf16_bits_to_f32, to_bf16_bits
    w = WORKLOADS["mixtral_fp8sq_dgrad_bf16"].replace(T=768, d=384, f=512, seed=6)
    print(f"[case] fp8 square scales {w}", flush=True)
    g = gen_all(w)
    rng = np.random.default_rng(12)

    def squares(m):
        E, R, C = m.shape
        s = np.exp2(rng.integers(-5, 6, (E, R // 32, C // 32))).astype(np.float32)
        return to_bf16_bits(bf16_bits_to_f32(m) * s.repeat(32, axis=1).repeat(32, axis=2))
    g["w13"], g["w2"] = squares(g["w13"]), squares(g["w2"])
    rep, flips, L, dev = run_and_compare(w, g)
    print(rep, flush=True)


# finegrained_small: many small groups; mixtral_small: every tile of the
# down-projection and dX GEMMs is split over K (few tiles per XCD), so the
# partial sums' arrival order varies between runs while the result must not
@pytest.mark.parametrize("name", ["finegrained_small", "mixtral_small"])
def test_determinism_bitwise(name):
    w = REDUCED[name]
    print(f"[case] determinism {w}", flush=True)
    import mixture_experts_layer_28_amd as moe
    g = gen_all(w)
    dev = {n: to_dev(v) for n, v in g.items()}
    outs = []
    for _ in range(2):
        L = moe.MoELayer(w.T, w.d, w.E, w.k, w.f, w.n_shared, w.dtype, w.score, w.act,
                         moe.capacity(w.T, w.k, w.E, w.cf), w.aux_coef, w.z_coef)
        L.step(dev)
        torch.cuda.synchronize()
        outs.append({n: bits(getattr(L, n)) for n in
                     ("topk_idx", "gate", "scores", "aux_out", "x_perm", "save_h", "out", "Y",
                      "dgate", "dx_perm", "dw13", "dw2", "dw_r", "dX")})
    for n in outs[0]:
        assert (outs[0][n] == outs[1][n]).all(), n


def test_zero_tokens():
    import mixture_experts_layer_28_amd as moe
    print("[case] zero tokens", flush=True)
    w = Workload("zero", T=0, d=64, E=4, k=2, f=64, n_shared=1)
    L = moe.MoELayer(w.T, w.d, w.E, w.k, w.f, w.n_shared, w.dtype, w.score, w.act, None, 0.0)
    L.dw13.fill_(1.0)
    L.dw2.fill_(1.0)
    L.dw_r.fill_(1.0)
    z = lambda *s, dt=torch.bfloat16: torch.ones(*s, dtype=dt, device="cuda")
    inp = dict(x=z(1, 64), w_r=z(4, 64, dt=torch.float32), w13=z(4, 128, 64), w2=z(4, 64, 64),
               sw13=z(1, 128, 64), sw2=z(1, 64, 64), dy=z(1, 64))
    L.step(inp)
    torch.cuda.synchronize()
    assert not L.dw13.float().any() and not L.dw2.float().any() and not L.dw_r.any()
    assert not L.dsw13.float().any()
