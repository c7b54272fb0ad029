"""bench.py's host logic, no GPU: the per-launch flop table against the
layer's totals, the FP8 launch classification and dtype labels, the traffic
guard (a counter summary taken on other GEMM sources or another workload is
not used), and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import bench
from moe_inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_gemm_flops_match_the_layer_totals():
    # SwiGLU: forward 6·A·d·f (up 2·A·d·2f, down 2·A·f·d); the backward is twice the forward
    w = WORKLOADS["mixtral_bf16"]
    A = 16384
    fl = bench.gemm_flops(w, A)
    assert fl["gemm_fwd_up"] + fl["gemm_fwd_down"] == 6 * A * w.d * w.f
    assert sum(fl.values()) == 18 * A * w.d * w.f
    # GELU (one up matrix): 4·A·d·f forward, 12·A·d·f in all
    g = WORKLOADS["skewed_bf16"]
    assert sum(bench.gemm_flops(g, 1000).values()) == 12 * 1000 * g.d * g.f
    # a shared expert adds T rows through every matrix
    s = WORKLOADS["dsv3_bf16"]
    assert sum(bench.gemm_flops(s, 65536).values()) == 18 * (65536 + s.T) * s.d * s.f


def test_fp8_launch_classification_and_labels():
    bf, f8, f8d = (WORKLOADS[n] for n in ("mixtral_bf16", "mixtral_fp8_bf16", "mixtral_fp8_dgrad_bf16"))
    roles = ["gemm_fwd_up", "gemm_fwd_down", "gemm_dgrad_down", "gemm_dgrad_up", "gemm_wgrad_down",
             "gemm_wgrad_up"]
    assert [bench.is_fp8_gemm(bf, r) for r in roles] == [False] * 6
    assert [bench.is_fp8_gemm(f8, r) for r in roles] == [True, True, False, False, False, False]
    assert [bench.is_fp8_gemm(f8d, r) for r in roles] == [True, True, True, True, False, False]
    assert bench.dtype_label(bf) == "bf16"
    assert bench.dtype_label(f8) == "fp8-e4m3 fwd GEMMs, bf16 bwd"
    assert bench.dtype_label(f8d) == "fp8-e4m3 fwd and dgrad GEMMs, bf16 wgrad"
    assert bench.dtype_label(WORKLOADS["tiny_fp32"]) == "f32"
    f8w = WORKLOADS["mixtral_fp8_all_bf16"]
    assert [bench.is_fp8_gemm(f8w, r) for r in roles] == [True] * 6
    assert bench.dtype_label(f8w) == "fp8-e4m3 fwd, dgrad and wgrad GEMMs (wgrad: 32-token block scales)"
    assert bench.dtype_label(WORKLOADS["mixtral_fp8b_bf16"]) == \
        "fp8-e4m3 fwd GEMMs (1x32 block scales), bf16 bwd"


def test_traffic_is_used_only_for_the_sources_and_workload_it_was_taken_on(monkeypatch):
    with open(bench.traffic_path("mixtral_bf16")) as fh:
        tr = json.load(fh)
    kernel = next(iter(tr["kernels"]))
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: tr["source_sha"])
    assert bench.traffic_for(kernel, tr["workload"]) == int(tr["kernels"][kernel]["bytes_per_launch"])
    # no summary for this workload; a summary taken on another workload
    assert bench.traffic_for(kernel, "top1_bf16") is None
    monkeypatch.setattr(bench, "traffic_path", lambda w: os.path.join(ROOT, "profiles",
                                                                       "traffic_mixtral_bf16.json"))
    assert bench.traffic_for(kernel, "finegrained_bf16") is None
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: "0" * 16)
    assert bench.traffic_for(kernel, tr["workload"]) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_streamed_cpu_baseline_equals_the_oracle_layer():
    """The CPU baseline streams the experts' weights one at a time; it must
    compute the same fwd+bwd as the oracle's whole-layer functions."""
    import numpy as np
    import oracle as O
    from moe_inputs import as_f64, gen_all
    for name, kw in (("dsv3_bf16", dict(T=64, d=32, f=16, E=12)),
                     ("mixtral_noisy_bf16", dict(T=48, d=32, f=24)),
                     ("skewed_bf16", dict(T=40, d=16, f=32))):
        w = WORKLOADS[name].replace(**kw)
        g = gen_all(w)
        clock = [0.0]
        got = bench.streamed_oracle_step(w, g, 32, clock)
        assert clock[0] > 0
        ws = w.replace(T=32)
        f = {n: (as_f64(v, w.dtype) if v is not None else None) for n, v in g.items()}
        x, dy = f["x"][:32], f["dy"][:32]
        gu = f["gumbel_u"][:32] if f["gumbel_u"] is not None else None
        cap = O.capacity(32, ws.k, ws.E, ws.cf)
        fwd = O.layer_forward(x, f["w_r"], f["w13"], f["w2"], ws.k, ws.score, ws.act, cap,
                              f["logit_bias"], f["sel_bias"], f["sw13"], f["sw2"], gu, ws.gumbel_tau)
        bwd = O.layer_backward(fwd, x, f["w_r"], f["w13"], f["w2"], dy, ws.score, ws.act,
                               ws.aux_coef, f["sw13"], f["sw2"], ws.z_coef, ws.gumbel_tau)
        np.testing.assert_allclose(got["Y"], fwd["Y"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(got["dX"], bwd["dX"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(got["dgate"], bwd["dgate"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(got["dw_r"], bwd["dw_r"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(got["dw_sums"][:, 0], bwd["dw13"].sum(axis=(1, 2)), atol=1e-9)
        np.testing.assert_allclose(got["dw_sums"][:, 1], bwd["dw2"].sum(axis=(1, 2)), atol=1e-9)


def test_gemm_roofline_picks_the_binding_bound():
    # DeepSeek-like weight gradient of the first matrix: 15 GB of bf16 dW13
    # written against 3.85 TFLOP, so HBM binds; the Mixtral-like dX GEMM is
    # matrix-core bound
    s = WORKLOADS["dsv3_bf16"]
    A = 65536
    fl, by = bench.gemm_flops(s, A), bench.gemm_bytes(s, A)
    assert by["gemm_wgrad_up"] == (A * 2 * s.f + A * s.d + s.E * 2 * s.f * s.d) * 2
    r = bench.gemm_roofline(s, "gemm_wgrad_up", fl["gemm_wgrad_up"], by["gemm_wgrad_up"], 4.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["frac"] - by["gemm_wgrad_up"] / 8e12 / 4e-3) < 1e-4
    assert r["attainable_frac"] == r["hbm_frac"] > r["mfma_frac"]
    m = WORKLOADS["mixtral_bf16"]
    fl, by = bench.gemm_flops(m, 16384), bench.gemm_bytes(m, 16384)
    r = bench.gemm_roofline(m, "gemm_dgrad_up", fl["gemm_dgrad_up"], by["gemm_dgrad_up"], 3.3)
    assert r["bound"] == "mfma" and abs(r["frac"] - fl["gemm_dgrad_up"] / 2.5e15 / 3.3e-3) < 1e-4


def test_kernel_base_name_and_trace_summary(tmp_path):
    assert bench.kernel_base_name("void moe::combine_kernel<unsigned short, 8>(unsigned short const*)") == \
        "combine_kernel"
    assert bench.kernel_base_name(
        "void moe::(anonymous namespace)::gemm_fp8_kernel<0, 1, true>(moe::GemmArgs)") == "gemm_fp8_kernel"
    w = WORKLOADS["mixtral_fp8_all_bf16"]
    roles = bench.gemm_roles(w)
    stats = tmp_path / "s.csv"
    trace = tmp_path / "t.csv"
    stats.write_text('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
                     '"void moe::(anonymous namespace)::gemm_fp8_kernel<0, 1, true>(moe::GemmArgs)",'
                     '12,12000,1000,90,900,1100,1\n')
    rows = ['"Kind","Dispatch_Id","Kernel_Name","Start_Timestamp","End_Timestamp"']
    did = 0
    for step in range(2):
        for i, _ in enumerate(roles):
            did += 1
            rows.append(f'"KERNEL_DISPATCH",{did},"void moe::(anonymous namespace)::gemm_fp8_kernel<0, 1, true>'
                        f'(moe::GemmArgs)",{did * 10**6},{did * 10**6 + 1000 * (i + 1)}')
            did += 1
            rows.append(f'"KERNEL_DISPATCH",{did},"moe::fill_zero_kernel(unsigned int*)",{did * 10**6},'
                        f'{did * 10**6 + 5}')
    trace.write_text("\n".join(rows) + "\n")
    out = tmp_path / "k.txt"
    bench.summarize_trace(str(stats), str(trace), w.name, out_path=str(out))
    text = out.read_text()
    # each role's launches averaged in launch order (role i took (i + 1) us here)
    for i, role in enumerate(roles):
        line = next(ln for ln in text.splitlines() if f" {role} " in ln)
        assert line.split()[0] == "2" and float(line.split()[1]) == 1.0 * (i + 1)
    assert "--summarize-trace" in text
