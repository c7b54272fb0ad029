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


def test_traffic_is_used_only_for_the_sources_and_workload_it_was_taken_on(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "gemm_traffic.json")) as fh:
        tr = json.load(fh)
    kernel = next(iter(tr["kernels"]))
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: tr["source_sha"])
    assert bench.traffic_for(kernel, tr["workload"]) == int(tr["kernels"][kernel]["bytes_per_launch"])
    assert bench.traffic_for(kernel, "finegrained_bf16") is None
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: "0" * 16)
    assert bench.traffic_for(kernel, tr["workload"]) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
