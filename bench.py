"""Benchmark one MoE layer step (forward + backward, every stage of the hot
path) on one MI355X, and print one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral_bf16]

A step = router, load-balance stats, permute, grouped FFN forward, combine,
combine backward, grouped FFN backward, router backward, un-permute, over
one batch of seeded synthetic inputs already resident in HBM. W untimed
steps, then K steps between two synchronisations. Per-kernel durations come
from the library's timing events (recorded on the launch stream) over the
same timed steps; the roofline object is for the dominant kernel. The CPU
oracle is timed on a bounded token sample of the same workload on the host
cores (rank 0, one GPU).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from moe_inputs import WORKLOADS, as_f64, gen_all  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 matrix peak
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "MoE layer fwd+bwd tokens/s on 1 MI355X; grouped-GEMM % bf16 MFMA peak"
GEMM_SOURCES = ("csrc/gemm_bf16.hip", "csrc/gemm_tile.h", "csrc/common.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_flops(w, A):
    """Algorithmic flops of each grouped-GEMM launch (only selected experts)."""
    P = 2 * w.f if w.act == "swiglu" else w.f
    d, f = w.d, w.f
    out = {
        "gemm_fwd_up": 2 * A * d * P, "gemm_fwd_down": 2 * A * f * d,
        "gemm_dgrad_down": 2 * A * d * f, "gemm_dgrad_up": 2 * A * P * d,
        "gemm_wgrad_down": 2 * A * d * f, "gemm_wgrad_up": 2 * A * P * d,
    }
    if w.n_shared:
        T = w.T
        out.update({
            "gemm_shared_fwd_up": 2 * T * d * P, "gemm_shared_fwd_down": 2 * T * f * d,
            "gemm_shared_dgrad_down": 2 * T * d * f, "gemm_shared_dgrad_up": 2 * T * P * d,
            "gemm_shared_wgrad_down": 2 * T * d * f, "gemm_shared_wgrad_up": 2 * T * P * d,
        })
    return out


def is_fp8_gemm(w, name):
    """Whether this grouped-GEMM launch runs on E4M3 operands."""
    return (w.fp8 and "fwd" in name) or (w.fp8_bwd and "dgrad" in name)


def dtype_label(w):
    if w.dtype != "bf16":
        return "f32"
    if w.fp8 and w.fp8_bwd:
        return "fp8-e4m3 fwd and dgrad GEMMs, bf16 wgrad"
    return "fp8-e4m3 fwd GEMMs, bf16 bwd" if w.fp8 else "bf16"


def hbm_bytes(w, A):
    """Algorithmic HBM bytes of the streaming stages (each tensor read or
    written once)."""
    s = 2 if w.dtype == "bf16" else 4
    T, d, k = w.T, w.d, w.k
    ns = T * d * s if w.n_shared else 0
    return {
        "permute": T * d * s + A * d * s + T * k * 4 * 3 + A * 4,
        "combine": A * d * s + T * d * s + ns + T * k * 8,
        "combine_bwd": T * d * s + 2 * A * d * s + T * k * 12,
        "unpermute": A * d * s + T * d * 4 + ns + T * d * s + T * k * 4,
    }


def gemm_source_hash():
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_layer_28_amd", rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, workload):
    """Measured HBM bytes per launch from the committed counter summary, if it
    was taken on the current GEMM sources; else None."""
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    try:
        with open(path) as fh:
            tr = json.load(fh)
    except (OSError, ValueError):
        return None
    if tr.get("source_sha") != gemm_source_hash() or tr.get("workload") != workload:
        return None
    k = tr.get("kernels", {}).get(kernel)
    return None if k is None else int(k["bytes_per_launch"])


def gemm_roles(w):
    """Order of the grouped-GEMM launches in one layer step (library call order)."""
    fwd = ["gemm_fwd_up", "gemm_fwd_down"]
    bwd = ["gemm_dgrad_down", "gemm_dgrad_up", "gemm_wgrad_down", "gemm_wgrad_up"]
    if w.n_shared:
        fwd += ["gemm_shared_" + r[5:] for r in fwd]
        bwd += ["gemm_shared_" + r[5:] for r in bwd]
    return fwd + bwd


CALIB_BYTES = 1 << 30   # plain device copy used to scale the HBM byte counters


def summarize_pmc(fetch_csv, write_csv, workload):
    """HBM bytes per launch of each grouped-GEMM role from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for the calibration copy of CALIB_BYTES (read once, written
    once). Writes profiles/gemm_traffic.json."""
    import csv
    w = WORKLOADS[workload]
    roles = gemm_roles(w)

    def load(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        # the calibration pass is the last multiply kernel before the layer's own
        calib = [float(r["Counter_Value"]) for r in rows
                 if "elementwise" in r["Kernel_Name"] and "Mul" in r["Kernel_Name"]]
        gem = [float(r["Counter_Value"]) for r in rows if "gemm_bf16_kernel" in r["Kernel_Name"]]
        per_role = {}
        for i, v in enumerate(gem):
            per_role.setdefault(roles[i % len(roles)], []).append(v)
        return calib, per_role

    fc, fr = load(fetch_csv, "FETCH_SIZE")
    wc, wr = load(write_csv, "WRITE_SIZE")
    if not fc or not wc:
        raise SystemExit("calibration copy not found in the counter files")
    f_scale = CALIB_BYTES / (fc[-1] * 1024.0)
    w_scale = CALIB_BYTES / (wc[-1] * 1024.0)
    out = {"workload": workload, "source_sha": gemm_source_hash(),
           "counters": "FETCH_SIZE, WRITE_SIZE (KiB per dispatch), two separate rocprofv3 --pmc runs; "
                       "$R = repository root, $OUT = a directory for the counter output",
           "commands": [
               "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE -d $OUT/pmc_fetch -o f "
               "--output-format csv -- python3 $R/bench.py --steps 2 --warmup 1 --no-cpu-baseline "
               "--no-profile --calibrate-copy",
               "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE -d $OUT/pmc_write -o w "
               "--output-format csv -- python3 $R/bench.py --steps 2 --warmup 1 --no-cpu-baseline "
               "--no-profile --calibrate-copy",
               "python bench.py --summarize-pmc $OUT/pmc_fetch/f_counter_collection.csv "
               "$OUT/pmc_write/w_counter_collection.csv"],
           "calibration": {"bytes": CALIB_BYTES, "fetch_kib": fc[-1], "write_kib": wc[-1],
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "kernels": {}}
    for role in roles:
        if role not in fr or role not in wr:
            continue
        fk = sum(fr[role]) / len(fr[role])
        wk = sum(wr[role]) / len(wr[role])
        out["kernels"][role] = {"fetch_kib": fk, "write_kib": wk,
                                "bytes_per_launch": int(fk * 1024 * f_scale + wk * 1024 * w_scale)}
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def gpu_clock_info():
    """GPU clocks and power limit as the vendor tool reports them (best effort;
    None where the tool is absent or refuses)."""
    import subprocess
    out = {}
    for key, cmd in (("metric", ["amd-smi", "metric", "-g", "0", "--clock", "--power", "--json"]),
                     ("limit", ["amd-smi", "static", "-g", "0", "--limit", "--json"])):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
            txt = r.stdout.strip()
            try:
                out[key] = json.loads(txt)
            except ValueError:
                out[key] = txt[-2000:] or None
        except (OSError, subprocess.SubprocessError):
            out[key] = None
    return out


def stage_detail(layer, inp, moe, w, A, iters=20):
    """Median time of each streaming stage as one C-ABI call, with and without a
    512 MiB write before every timed call (that write evicts the 256 MB MALL, so
    the flushed figure reads its inputs from HBM), and a per-expert loop of
    torch's own GEMM (hipBLASLt) on the two forward shapes, as context."""
    import torch
    import torch.nn.functional as F
    D = layer.desc
    x, dy = inp["x"], inp["dy"]
    calls = {
        "permute": lambda: moe.permute(D, x, layer.topk_idx, layer.offsets, layer.row_of,
                                       layer.token_of, layer.n_dropped, layer.x_perm, layer.ws),
        "combine": lambda: moe.combine(D, layer.out, layer.out_shared, layer.gate, layer.row_of,
                                       layer.Y),
        "combine_bwd": lambda: moe.combine_bwd(D, dy, layer.out, layer.gate, layer.row_of,
                                               layer.dgate, layer.dout),
        "unpermute": lambda: moe.permute_bwd(D, layer.dx_perm, layer.row_of, layer.dx_shared,
                                             layer.dx_router, layer.dX),
    }
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def median_ms(fn, flushed):
        ts = []
        for i in range(iters + 2):
            if flushed:
                flush.fill_(i & 0xFF)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            if i >= 2:
                ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    hb = hbm_bytes(w, A)
    out = {}
    for name, fn in calls.items():
        r = {}
        for tag, fl in (("unflushed", False), ("flushed", True)):
            ms = median_ms(fn, fl)
            gbs = hb[name] / (ms / 1e3) / 1e9
            r[tag] = {"median_ms": round(ms, 4), "GB/s": round(gbs, 1),
                      "hbm_frac": round(gbs / PEAK_HBM_GBS, 3)}
        out[name] = r
    # context only: torch's GEMM per expert, same operands as the forward launches
    off = layer.offsets.cpu().tolist()
    w13, w2 = inp["w13"], inp["w2"]
    H = layer.save_h
    up = lambda: [F.linear(layer.x_perm[off[e]:off[e + 1]], w13[e]) for e in range(w.E)]
    down = lambda: [F.linear(H[off[e]:off[e + 1]], w2[e]) for e in range(w.E)]
    fl = gemm_flops(w, A)
    cmp_ = {}
    for name, fn in (("gemm_fwd_up", up), ("gemm_fwd_down", down)):
        ms = median_ms(fn, False)
        cmp_[name] = {"median_ms": round(ms, 4), "TFLOP/s": round(fl[name] / (ms / 1e3) / 1e12, 1),
                      "note": "torch.nn.functional.linear per expert (hipBLASLt), no fused "
                              "epilogue; context, not part of the library"}
    del flush
    return {"iters": iters, "stages": out, "torch_gemm_per_expert": cmp_,
            "gpu_clocks": gpu_clock_info()}


def cpu_baseline(w, g, tokens):
    """The oracle, as it stands, on the first `tokens` tokens of the workload
    (same weights; capacity recomputed for the sample)."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    ws = w.replace(T=tokens)
    f = {n: (as_f64(v, w.dtype) if v is not None else None) for n, v in g.items()}
    x, dy = f["x"][:tokens], f["dy"][:tokens]
    gu = f["gumbel_u"][:tokens] if f["gumbel_u"] is not None else None
    cap = O.capacity(ws.T, ws.k, ws.E, ws.cf)
    t0 = time.perf_counter()
    fwd = O.layer_forward(x, f["w_r"], f["w13"], f["w2"], ws.k, ws.score, ws.act, cap,
                          f["logit_bias"], f["sel_bias"], f["sw13"], f["sw2"], gu, ws.gumbel_tau,
                          fp8=ws.fp8)
    O.layer_backward(fwd, x, f["w_r"], f["w13"], f["w2"], dy, ws.score, ws.act, ws.aux_coef,
                     f["sw13"], f["sw2"], ws.z_coef, ws.gumbel_tau, fp8_dgrad=ws.fp8_bwd)
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {tokens} of {w.T} tokens, all {w.E} experts' weights, fwd+bwd in "
                      f"float64 NumPy ({dt:.1f} s; bf16->float64 input conversion untimed)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixtral_bf16", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true",
                    help="time without per-kernel events (roofline object omitted)")
    ap.add_argument("--stage-detail", action="store_true",
                    help="also time each streaming stage alone, MALL-flushed and not, "
                         "torch's per-expert GEMM as context, and record GPU clocks")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 1 GiB device copy first (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/gemm_traffic.json from two counter runs and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import mixture_experts_layer_28_amd as moe
    from mixture_experts_layer_28_amd import MoELayer

    w = WORKLOADS[args.workload]
    log(f"[bench] workload {w}")
    t0 = time.perf_counter()
    g = gen_all(w)
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s")

    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    inp = {n: dev(v) for n, v in g.items()}
    if args.calibrate_copy:
        # one elementwise pass reading and writing CALIB_BYTES each
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    cap = moe.capacity(w.T, w.k, w.E, w.cf)
    layer = MoELayer(w.T, w.d, w.E, w.k, w.f, w.n_shared, w.dtype, w.score, w.act, cap,
                     w.aux_coef, w.z_coef, w.bias_gamma, w.gumbel_tau or 0.0, fp8_fwd=w.fp8,
                     fp8_bwd=w.fp8_bwd)
    for _ in range(args.warmup):
        layer.step(inp)
    torch.cuda.synchronize()
    log("[bench] warmup done")

    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if not args.no_profile:
        moe.profile_enable(True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        layer.step(inp)
    ev1.record(stream)
    torch.cuda.synchronize()
    prof = moe.profile_read() if not args.no_profile else []
    moe.profile_enable(False)
    ms = ev0.elapsed_time(ev1)
    ms_step = ms / args.steps
    value = w.T * args.steps / (ms / 1e3)
    A = int(layer.offsets[-1].item())
    log(f"[bench] {ms_step:.3f} ms/step, {value:.0f} tokens/s, kept rows {A}")

    flops = gemm_flops(w, A)
    stages = {}
    for name, tot, n in prof:
        stages[name] = {"avg_ms": round(tot / n, 4), "launches": n}
    roofline = None
    gemm_tot_ms = sum(tot for name, tot, n in prof if name in flops)
    gemm_flops_step = sum(flops.values())
    if prof:
        gk = [(tot, name, n) for name, tot, n in prof if name in flops]
        tot, dom, n = max(gk)
        avg_s = tot / n / 1e3
        achieved = flops[dom] / avg_s / 1e12
        fp8_kernel = is_fp8_gemm(w, dom)
        peak = (PEAK_FP8_TFLOPS if fp8_kernel else PEAK_BF16_TFLOPS) if w.dtype == "bf16" \
            else PEAK_F32_TFLOPS
        roofline = {"bound": "mfma" if w.dtype == "bf16" else "alu", "kernel": dom,
                    "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4),
                    "traffic": traffic_for(dom, w.name),
                    "flops_per_launch": flops[dom], "avg_ms": round(tot / n, 4)}
        if fp8_kernel:
            roofline["operand_dtype"] = "fp8-e4m3"
        hb = hbm_bytes(w, A)
        for name, b in hb.items():
            if name in stages:
                gbs = b / (stages[name]["avg_ms"] / 1e3) / 1e9
                stages[name]["GB/s"] = round(gbs, 1)
                stages[name]["hbm_frac"] = round(gbs / PEAK_HBM_GBS, 3)
        for name in flops:
            if name in stages:
                tf = flops[name] / (stages[name]["avg_ms"] / 1e3) / 1e12
                stages[name]["TFLOP/s"] = round(tf, 1)
    gemm_tflops = gemm_flops_step * args.steps / (gemm_tot_ms / 1e3) / 1e12 if gemm_tot_ms else None
    # share of the matrix peak: time the GEMMs would take at their operand
    # dtype's peak (fp8 forward GEMMs at the fp8 peak) over the time they took
    mfma_frac = None
    if gemm_tot_ms and w.dtype == "bf16":
        ideal_s = sum(flops[name] * n / ((PEAK_FP8_TFLOPS if is_fp8_gemm(w, name)
                                          else PEAK_BF16_TFLOPS) * 1e12)
                      for name, tot, n in prof if name in flops)
        mfma_frac = ideal_s / (gemm_tot_ms / 1e3)

    detail = None
    if args.stage_detail:
        log("[bench] stage detail (flushed / unflushed, torch GEMM context, clocks)")
        detail = stage_detail(layer, inp, moe, w, A)
        log("[bench] stage detail done")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle on {args.cpu_tokens} tokens")
        cpu = cpu_baseline(w, g, args.cpu_tokens)
        log(f"[bench] oracle: {cpu['value']:.2f} tokens/s")

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_label(w), "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "E": w.E, "k": w.k, "f": w.f,
                   "act": w.act, "score": w.score, "n_shared": w.n_shared,
                   "capacity": cap, "kept_rows": A, "fp8_fwd": w.fp8, "fp8_dgrad": w.fp8_bwd,
                   "parallelism": "none (1 GPU)"},
        "gemm_tflops": round(gemm_tflops, 1) if gemm_tflops else None,
        "gemm_mfma_frac": round(mfma_frac, 4) if mfma_frac else None,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stages": stages,
    }
    if detail is not None:
        out["stage_detail"] = detail
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
