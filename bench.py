"""Benchmark one MoE layer step (forward + backward, every stage of the hot
path) on one MI355X, and print one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3_bf16]

A step = router, load-balance stats, permute, grouped FFN forward, combine,
combine backward, grouped FFN backward, router backward, un-permute, over
one batch of seeded synthetic inputs already resident in HBM. The default
workload is the largest configuration, the DeepSeek-like layer (dsv3_bf16).
W untimed steps, then K timed steps between two synchronisations (the
headline; one event between consecutive steps gives the median step). A
second, profiled pass of K steps records the library's timing events
around every kernel launch (on the launch stream) for the per-kernel times
and the roofline object of the dominant kernel. The CPU oracle is timed on a
bounded token sample of the same workload on the host cores (rank 0, one
GPU), streaming the experts' weights one at a time.
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


def gemm_bytes(w, A):
    """Algorithmic HBM bytes of each grouped-GEMM launch: every operand read
    once and every output written once (all E experts' weights, and their
    gradients, whatever their row counts)."""
    s = 2 if w.dtype == "bf16" else 4
    P = 2 * w.f if w.act == "swiglu" else w.f
    d, f, E = w.d, w.f, w.E

    def roles(R, G):
        return {
            "fwd_up": (R * d + G * P * d + R * f + R * P) * s,
            "fwd_down": (R * f + G * d * f + R * d) * s,
            "dgrad_down": (R * d + G * d * f + R * P + R * P) * s,
            "dgrad_up": (R * P + G * P * d + R * d) * s,
            "wgrad_down": (R * d + R * f + G * d * f) * s,
            "wgrad_up": (R * P + R * d + G * P * d) * s,
        }
    out = {"gemm_" + k: v for k, v in roles(A, E).items()}
    if w.n_shared:
        out.update({"gemm_shared_" + k: v for k, v in roles(w.T, 1).items()})
    return out


def gemm_roofline(w, name, flops, nbytes, avg_ms):
    """Roofline of one grouped-GEMM launch: the matrix-core time (flops at the
    operand dtype's peak) and the HBM time (algorithmic bytes at 8 TB/s); the
    larger one binds. frac = achieved / peak of the binding roofline;
    mfma_frac and hbm_frac are each ideal time over the measured time, and
    attainable_frac = max of the two."""
    fp8_kernel = is_fp8_gemm(w, name)
    peak_f = (PEAK_FP8_TFLOPS if fp8_kernel else PEAK_BF16_TFLOPS) if w.dtype == "bf16" \
        else PEAK_F32_TFLOPS
    t = avg_ms / 1e3
    t_mfma = flops / (peak_f * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_hbm > t_mfma:
        out = {"bound": "hbm", "achieved": round(nbytes / t / 1e9, 1), "peak": PEAK_HBM_GBS,
               "unit": "GB/s", "frac": round(t_hbm / t, 4)}
    else:
        out = {"bound": "mfma" if w.dtype == "bf16" else "alu",
               "achieved": round(flops / t / 1e12, 1), "peak": peak_f, "unit": "TFLOP/s",
               "frac": round(t_mfma / t, 4)}
    out.update({"kernel": name, "avg_ms": round(avg_ms, 4), "flops_per_launch": flops,
                "bytes_per_launch": nbytes, "tflops": round(flops / t / 1e12, 1),
                "mfma_frac": round(t_mfma / t, 4), "hbm_frac": round(t_hbm / t, 4),
                "attainable_frac": round(max(t_mfma, t_hbm) / t, 4)})
    if fp8_kernel:
        out["operand_dtype"] = "fp8-e4m3"
    return out


def is_fp8_gemm(w, name):
    """Whether this grouped-GEMM launch runs on E4M3 operands."""
    return ((w.fp8 and "fwd" in name) or (w.fp8_bwd and "dgrad" in name)
            or (w.fp8_wgrad and "wgrad" in name))


def dtype_label(w):
    if w.dtype != "bf16":
        return "f32"
    blk = {"block": " (1x32 block scales)",
           "square": " (32x32 weight squares, 1x32 activation blocks)"}.get(w.fp8_scale, "")
    if w.fp8 and w.fp8_bwd and w.fp8_scale == "square":
        wg = " and wgrad GEMMs (wgrad: 32-token block scales)" if w.fp8_wgrad else " GEMMs, bf16 wgrad"
        return f"fp8-e4m3 fwd and dgrad{blk}{wg}"
    if w.fp8 and w.fp8_wgrad:
        return f"fp8-e4m3 fwd{blk}, dgrad and wgrad GEMMs (wgrad: 32-token block scales)"
    if w.fp8 and w.fp8_bwd:
        return f"fp8-e4m3 fwd{blk} and dgrad GEMMs, bf16 wgrad"
    return f"fp8-e4m3 fwd GEMMs{blk}, bf16 bwd" if w.fp8 else "bf16"


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


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def traffic_for(kernel, workload):
    """Measured HBM bytes per launch from the committed counter summary of this
    workload, if it was taken on the current GEMM sources; else None."""
    path = traffic_path(workload)
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

# streaming stages: the kernels each one launches (function names as the
# profiler prints them) and its algorithmic bytes (hbm_bytes)
STREAM_KERNELS = {"permute": ("perm_count_kernel", "perm_gather_kernel"),
                  "combine": ("combine_kernel",), "combine_bwd": ("combine_bwd_kernel",),
                  "unpermute": ("unpermute_kernel",)}


def kernel_base_name(name):
    """'void moe::combine_kernel<unsigned short, 8>(...)' -> 'combine_kernel'
    (also inside an anonymous namespace)."""
    head = name.replace("(anonymous namespace)::", "").split("(")[0].split("<")[0].strip()
    return head.split("::")[-1].split()[-1]


def trace_path(workload):
    return os.path.join(ROOT, "profiles", f"kernel_stats_{workload}.txt")


def is_grouped_gemm(name):
    """A launch of one of the layer's grouped GEMMs (bf16 or FP8 kernel),
    not one of the router's float32-output products on the bf16 kernel
    (epilogue 5, gemm_bf16_kernel<5, ...>)."""
    return ("gemm_bf16_kernel" in name and "gemm_bf16_kernel<5," not in name) or "gemm_fp8_kernel" in name


def summarize_trace(stats_csv, trace_csv, workload, out_path=None):
    """Text summary of a rocprofv3 --kernel-trace --stats run of this
    workload's bench (TRACE_COMMAND): every kernel's calls and durations, then
    the grouped-GEMM launches by role (the library launches them in
    gemm_roles order once per step), so a role's average duration can be set
    against the bench's stage of the same name. Writes
    profiles/kernel_stats_<workload>.txt unless out_path is given."""
    import csv
    w = WORKLOADS[workload]
    stats = sorted(csv.DictReader(open(stats_csv)), key=lambda r: -float(r["TotalDurationNs"]))
    disp = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Dispatch_Id"]))
    gem = [r for r in disp if is_grouped_gemm(r["Kernel_Name"])
           or (w.dtype == "fp32" and "gemm_f32_mfma_kernel" in r["Kernel_Name"]
               and "GemmArgs" in r["Kernel_Name"])]
    roles = gemm_roles(w)
    per_role = {}
    for i, r in enumerate(gem):
        ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        per_role.setdefault(roles[i % len(roles)], []).append((ns, kernel_base_name(r["Kernel_Name"])))
    cmd = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d $OUT/trace -o t "
           f"--output-format csv -- python3 $R/bench.py --workload {workload} --steps 5 --warmup 2 "
           "--no-cpu-baseline --no-profile")
    lines = [f"# rocprofv3 kernel trace summary: MoE layer fwd+bwd, {workload} workload "
             f"(bench.py --workload {workload}), 2 warmup + 5 timed steps",
             "# command (on the MI355X, repo root = $R, $OUT = an output directory):",
             f"#   {cmd}",
             f"# summarized by: python bench.py --workload {workload} --summarize-trace "
             "$OUT/trace/t_kernel_stats.csv $OUT/trace/t_kernel_trace.csv", "",
             "## kernels (from t_kernel_stats.csv, all steps of the run)",
             " calls     avg_us     min_us     max_us   total_ms    pct  kernel"]
    for r in stats:
        lines.append("%6d %10.1f %10.1f %10.1f %10.2f %6.2f  %s" % (
            int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"]), r["Name"][:110]))
    if gem:
        lines += ["", "## grouped-GEMM launches by role (from t_kernel_trace.csv, in launch order per step; "
                  f"{len(gem)} launches = {len(gem) / len(roles):g} steps x {len(roles)} roles)",
                  " calls     avg_us     min_us     max_us  role                     kernel"]
        for role in roles:
            v = per_role.get(role, [])
            if not v:
                continue
            ds = [ns / 1e3 for ns, _ in v]
            lines.append("%6d %10.1f %10.1f %10.1f  %-24s %s" % (len(ds), sum(ds) / len(ds), min(ds), max(ds),
                                                              role, v[0][1]))
    path = out_path or trace_path(workload)
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(path)


MFMA_COMMAND = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc MfmaUtil SQ_VALU_MFMA_BUSY_CYCLES "
                "GRBM_GUI_ACTIVE -d $OUT/pmc_mfma_<workload> -o m --output-format csv -- python3 "
                "$R/bench.py --workload <workload> --steps 2 --warmup 1 --no-cpu-baseline --no-profile")


def summarize_mfma(out_path, pairs):
    """MFMA busy share and shader clock of each grouped-GEMM launch of the last
    step, from one rocprofv3 --pmc run per workload (MFMA_COMMAND); pairs =
    [(workload, counter_csv), ...]. MfmaUtil is rocprofv3's derived counter
    (sum of SQ_VALU_MFMA_BUSY_CYCLES over max GRBM_GUI_ACTIVE times the SIMD
    count, in %); the clock is GRBM_GUI_ACTIVE summed over the 8 XCDs / 8 / the
    dispatch's duration."""
    import csv
    lines = ["# MFMA busy share and clock per grouped-GEMM launch (rocprofv3 derived counter MfmaUtil =",
             "#   sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) * SIMD count) * 100; clock = GRBM_GUI_ACTIVE",
             "#   (summed over the 8 XCDs) / 8 / the dispatch's duration from the same record)",
             "# command (on the MI355X, repo root = $R, $OUT = an output directory), once per workload:",
             f"#   {MFMA_COMMAND}",
             "# summarized by: python bench.py --summarize-mfma OUT.txt <workload> $OUT/pmc_mfma_<workload>/"
             "m_counter_collection.csv ...",
             "# last step's grouped-GEMM launches, in launch order"]
    for workload, path in pairs:
        by = {}
        for r in csv.DictReader(open(path)):
            by.setdefault(int(r["Dispatch_Id"]), {})[r["Counter_Name"]] = r
        gem = [by[k] for k in sorted(by)
               if "GRBM_GUI_ACTIVE" in by[k] and is_grouped_gemm(by[k]["GRBM_GUI_ACTIVE"]["Kernel_Name"])]
        roles = gemm_roles(WORKLOADS[workload])
        last = gem[-len(roles):]
        lines += ["", f"## {workload}", "launch                 MfmaUtil %   clock MHz   duration us"]
        for role, d in zip(roles, last):
            g = d["GRBM_GUI_ACTIVE"]
            dur = (int(g["End_Timestamp"]) - int(g["Start_Timestamp"])) / 1e3
            clk = float(g["Counter_Value"]) / 8 / (dur * 1e-6) / 1e6
            lines.append("%-22s %10.1f %11.0f %13.1f" % (role, float(d["MfmaUtil"]["Counter_Value"]), clk, dur))
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(out_path)


def summarize_pmc(fetch_csv, write_csv, workload, stats_csv=None):
    """HBM bytes per launch of each grouped-GEMM role and streaming stage from
    two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each
    scaled by what the same counter reads for the calibration copy of
    CALIB_BYTES (read once, written once). With a rocprofv3 --stats kernel
    summary, the streaming stages also get their counted bytes over their
    average duration (GB/s). Writes profiles/traffic_<workload>.json."""
    import csv
    w = WORKLOADS[workload]
    roles = gemm_roles(w)

    def load(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        # the calibration pass is the last multiply kernel before the layer's own
        calib = [float(r["Counter_Value"]) for r in rows
                 if "elementwise" in r["Kernel_Name"] and "Mul" in r["Kernel_Name"]]
        gem = [float(r["Counter_Value"]) for r in rows if is_grouped_gemm(r["Kernel_Name"])]
        per_role = {}
        for i, v in enumerate(gem):
            per_role.setdefault(roles[i % len(roles)], []).append(v)
        per_kernel = {}
        for r in rows:
            per_kernel.setdefault(kernel_base_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return calib, per_role, per_kernel

    # kept rows: every assignment without a capacity limit (else data-dependent)
    A = w.T * w.k if w.cf is None else None
    fc, fr, fk_all = load(fetch_csv, "FETCH_SIZE")
    wc, wr, wk_all = load(write_csv, "WRITE_SIZE")
    if not fc or not wc:
        raise SystemExit("calibration copy not found in the counter files")
    f_scale = CALIB_BYTES / (fc[-1] * 1024.0)
    w_scale = CALIB_BYTES / (wc[-1] * 1024.0)
    out = {"workload": workload, "source_sha": gemm_source_hash(),
           "counters": "FETCH_SIZE, WRITE_SIZE (KiB per dispatch), two separate rocprofv3 --pmc runs; "
                       "$R = repository root, $OUT = a directory for the counter output",
           "commands": [
               "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE -d $OUT/pmc_fetch -o f "
               f"--output-format csv -- python3 $R/bench.py --workload {workload} --steps 2 --warmup 1 "
               "--no-cpu-baseline --no-profile --calibrate-copy",
               "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE -d $OUT/pmc_write -o w "
               f"--output-format csv -- python3 $R/bench.py --workload {workload} --steps 2 --warmup 1 "
               "--no-cpu-baseline --no-profile --calibrate-copy",
               "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d $OUT/trace -o t "
               f"--output-format csv -- python3 $R/bench.py --workload {workload} --steps 5 --warmup 2 "
               "--no-cpu-baseline --no-profile",
               f"python bench.py --workload {workload} --summarize-pmc "
               "$OUT/pmc_fetch/f_counter_collection.csv $OUT/pmc_write/w_counter_collection.csv "
               "$OUT/trace/t_kernel_stats.csv"],
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
        if A is not None:
            out["kernels"][role]["algorithmic_bytes"] = gemm_bytes(w, A)[role]
    stats = {}
    if stats_csv:
        for r in csv.DictReader(open(stats_csv)):
            stats.setdefault(kernel_base_name(r["Name"]), []).append(float(r["AverageNs"]))
    out["streaming"] = {}
    for stage, kernels in STREAM_KERNELS.items():
        if not all(k in fk_all and k in wk_all for k in kernels):
            continue
        byt = sum(sum(fk_all[k]) / len(fk_all[k]) * 1024 * f_scale
                  + sum(wk_all[k]) / len(wk_all[k]) * 1024 * w_scale for k in kernels)
        rec = {"kernels": list(kernels), "bytes_per_launch": int(byt)}
        if A is not None:
            rec["algorithmic_bytes"] = hbm_bytes(w, A)[stage]
        if all(k in stats for k in kernels):
            ns = sum(sum(stats[k]) / len(stats[k]) for k in kernels)
            rec["avg_us"] = round(ns / 1e3, 2)
            rec["counted_GB/s"] = round(byt / ns, 1)
            rec["counted_hbm_frac"] = round(byt / ns / PEAK_HBM_GBS, 3)
        out["streaming"][stage] = rec
    path = traffic_path(workload)
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
    512 MiB read before every timed call (that read evicts the 256 MB MALL, so
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
    # the flush reads 512 MiB (twice the MALL) and writes 4 bytes: no dirty
    # lines of its own can be written back inside the timed call
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def median_ms(fn, flushed):
        ts = []
        for i in range(iters + 2):
            if flushed:
                flush.max()
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


# token sample of the CPU oracle per workload (about 10-30 s of float64 work
# on a 16-core host); other workloads use DEFAULT_CPU_TOKENS
CPU_TOKENS = {"dsv3_bf16": 4096, "finegrained_bf16": 2048, "mixtral_bf16": 4096}
DEFAULT_CPU_TOKENS = 2048


def cpu_baseline(w, g, tokens):
    """The oracle, as it stands, on the first `tokens` tokens of the workload
    (same weights; capacity recomputed for the sample), fwd+bwd in float64.

    The experts are streamed: each expert's bf16 weights are widened to
    float64 just before its rows run (untimed) and dropped after, so the
    host never holds every expert in float64 (about 90 GB for the
    DeepSeek-like layer). Per expert the oracle's own functions run on that
    expert's rows: expert_forward, combine_backward of those rows (their dO
    depends only on gates and dY) and expert_backward. Router, statistics,
    permutation, combine, router backward and un-permute run once on the
    whole sample. Only the oracle calls are timed."""
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    clock = [0.0]
    streamed_oracle_step(w, g, tokens, clock)
    dt_s = clock[0]
    return {"value": tokens / dt_s, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "blas_threads": blas,
            "sample": f"first {tokens} of {w.T} tokens (capacity recomputed for the sample), "
                      f"all {w.E} experts' weights streamed one expert at a time, fwd+bwd in "
                      f"float64 NumPy: {dt_s:.1f} s of oracle calls; bf16->float64 widening "
                      f"untimed"}


def streamed_oracle_step(w, g, tokens, clock):
    """One fwd+bwd of the oracle on the first `tokens` tokens, one expert's
    weights in float64 at a time (see cpu_baseline). Adds the seconds spent in
    oracle calls to clock[0]. Returns Y, dX, dgate, dw_r and, per expert, the
    sums of dW13 and dW2 (the weight gradients themselves are dropped with the
    expert's weights)."""
    import oracle as O
    ws = w.replace(T=tokens)
    dt = w.dtype
    cv = lambda a: as_f64(a, dt) if a is not None else None   # noqa: E731
    x, dy = cv(g["x"][:tokens]), cv(g["dy"][:tokens])
    w_r = g["w_r"].astype(np.float64)
    lb = g["logit_bias"].astype(np.float64) if g["logit_bias"] is not None else None
    sb = g["sel_bias"].astype(np.float64) if g["sel_bias"] is not None else None
    gu = g["gumbel_u"][:tokens].astype(np.float64) if g["gumbel_u"] is not None else None
    cap = O.capacity(ws.T, ws.k, ws.E, ws.cf)

    def timed(fn, *a):
        t0 = time.perf_counter()
        out = fn(*a)
        clock[0] += time.perf_counter() - t0
        return out

    def fwd_e(X, w13e, w2e):
        if ws.fp8 and ws.fp8_scale == "square":
            return O.expert_forward_fp8_square(X, w13e, w2e, ws.act)
        if ws.fp8 and ws.fp8_scale == "block":
            return O.expert_forward_fp8_block(X, w13e, w2e, ws.act)
        if ws.fp8:
            return O.expert_forward_fp8(X, w13e, w2e, ws.act)
        return O.expert_forward(X, w13e, w2e, ws.act)

    def bwd_e(X, w13e, w2e, sv, dO):
        if ws.fp8_bwd and ws.fp8_scale == "square":
            out = O.expert_backward_fp8_wq(X, O.quantize_weights_fp8_square(w2e).T,
                                           O.quantize_weights_fp8_square(w13e).T, sv, dO, ws.act,
                                           ws.fp8_grad, "block")
        elif ws.fp8_bwd:
            out = O.expert_backward_fp8_wq(X, O.quantize_weights_fp8_t(w2e),
                                           O.quantize_weights_fp8_t(w13e), sv, dO, ws.act, ws.fp8_grad)
        else:
            out = O.expert_backward(X, w13e, w2e, sv, dO, ws.act)
        if ws.fp8_wgrad:
            g13, g2 = O.expert_wgrad_fp8(X, sv["H"], dO, out[3], ws.fp8_grad)
            out = (out[0], g13, g2, out[3])
        return out

    r = timed(O.router_forward, x, w_r, ws.k, ws.score, lb, sb, gu, ws.gumbel_tau)
    st = timed(O.aux_stats, r["scores"], r["topk_idx"], ws.E)
    pm = timed(O.permute, r["topk_idx"], ws.E, cap)
    off, tok = pm["offsets"], pm["token_of"]
    A = int(off[-1])
    x_perm = timed(lambda: x[tok])
    Orows = np.zeros((A, ws.d))
    dX_perm = np.zeros((A, ws.d))
    dgate = np.zeros((ws.T, ws.k))
    slot_of = np.zeros(A, dtype=np.int64)
    kept = np.nonzero(pm["row_of"] >= 0)
    slot_of[pm["row_of"][kept]] = kept[1]
    gsum = np.zeros((ws.E, 2))
    for e in range(ws.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        w13e, w2e = cv(g["w13"][e]), cv(g["w2"][e])           # untimed widening
        te, je = tok[lo:hi], slot_of[lo:hi]
        o, sv = timed(fwd_e, x_perm[lo:hi], w13e, w2e)
        Orows[lo:hi] = o
        dg_e, dO_e = timed(O.combine_backward, dy[te], o, r["gates"][te, je][:, None],
                           np.arange(hi - lo)[:, None])
        dgate[te, je] = dg_e[:, 0]
        dxe, g13, g2, _ = timed(bwd_e, x_perm[lo:hi], w13e, w2e, sv, dO_e)
        dX_perm[lo:hi] = dxe
        gsum[e] = g13.sum(), g2.sum()
        del w13e, w2e, g13, g2
    Os = dXs = None
    if ws.n_shared:
        sw13, sw2 = cv(g["sw13"][0]), cv(g["sw2"][0])
        Os, svs = timed(fwd_e, x, sw13, sw2)
        dXs, _, _, _ = timed(bwd_e, x, sw13, sw2, svs, dy)
        del sw13, sw2
    Y = timed(O.combine, Orows, r["gates"], pm["row_of"], Os)
    rb = timed(O.router_backward, x, w_r, r["scores"], r["topk_idx"], r["gates"], dgate, ws.score,
               ws.aux_coef, st["y"], ws.z_coef, r["logits"], ws.gumbel_tau)
    dX = timed(O.permute_backward, dX_perm, pm["row_of"], dXs, rb["dx_router"])
    return dict(Y=Y, dX=dX, dgate=dgate, dw_r=rb["dw_r"], dw_sums=gsum)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dsv3_bf16", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="token sample of the CPU oracle (default: per workload, CPU_TOKENS)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true",
                    help="skip the profiled pass (no per-kernel times, roofline object omitted)")
    ap.add_argument("--stage-detail", action="store_true",
                    help="also time each streaming stage alone, MALL-flushed and not, "
                         "torch's per-expert GEMM as context, and record GPU clocks")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 1 GiB device copy first (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="CSV",
                    help="FETCH_CSV WRITE_CSV [KERNEL_STATS_CSV]: write "
                         "profiles/traffic_<workload>.json from two counter runs and exit")
    ap.add_argument("--summarize-trace", nargs=2, metavar="CSV",
                    help="KERNEL_STATS_CSV KERNEL_TRACE_CSV: write profiles/kernel_stats_<workload>.txt "
                         "from a rocprofv3 --kernel-trace --stats run and exit")
    ap.add_argument("--summarize-mfma", nargs="+", metavar="ARG",
                    help="OUT_TXT WORKLOAD CSV [WORKLOAD CSV ...]: MFMA busy share per grouped-GEMM "
                         "launch from rocprofv3 --pmc MfmaUtil runs, and exit")
    args = ap.parse_args()
    if args.summarize_mfma:
        sm = args.summarize_mfma
        if len(sm) < 3 or len(sm) % 2 == 0:
            ap.error("--summarize-mfma takes OUT_TXT followed by WORKLOAD CSV pairs")
        summarize_mfma(sm[0], list(zip(sm[1::2], sm[2::2])))
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace[0], args.summarize_trace[1], args.workload)
        return
    if args.summarize_pmc:
        if len(args.summarize_pmc) not in (2, 3):
            ap.error("--summarize-pmc takes FETCH_CSV WRITE_CSV [KERNEL_STATS_CSV]")
        pm = args.summarize_pmc
        summarize_pmc(pm[0], pm[1], args.workload, pm[2] if len(pm) == 3 else None)
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
                     fp8_bwd=w.fp8_bwd, fp8_scale=w.fp8_scale, fp8_wgrad=w.fp8_wgrad)
    for _ in range(args.warmup):
        layer.step(inp)
    torch.cuda.synchronize()
    log("[bench] warmup done")

    stream = torch.cuda.current_stream()
    # timed pass (the headline): K steps between two synchronisations, with
    # one timing event between consecutive steps and none inside a step
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(args.steps):
        layer.step(inp)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1])
    step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    ms_step = ms / args.steps
    value = w.T * args.steps / (ms / 1e3)
    A = int(layer.offsets[-1].item())
    log(f"[bench] {ms_step:.3f} ms/step (median {np.median(step_ms):.3f}), {value:.0f} tokens/s, "
        f"kept rows {A}")

    # profiled pass: the same K steps again with the library's timing events
    # around every kernel launch (per-kernel times, roofline)
    prof, prof_ms_step = [], None
    if not args.no_profile:
        moe.profile_enable(True)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            layer.step(inp)
        e1.record(stream)
        torch.cuda.synchronize()
        prof = moe.profile_read()
        moe.profile_enable(False)
        prof_ms_step = e0.elapsed_time(e1) / args.steps
        log(f"[bench] profiled pass: {prof_ms_step:.3f} ms/step")

    flops = gemm_flops(w, A)
    gbytes = gemm_bytes(w, A)
    stages = {}
    for name, tot, n in prof:
        stages[name] = {"avg_ms": round(tot / n, 4), "launches": n}
    roofline = None
    gemm_tot_ms = sum(tot for name, tot, n in prof if name in flops)
    gemm_flops_step = sum(flops.values())
    if prof:
        gk = [(tot, name, n) for name, tot, n in prof if name in flops]
        tot, dom, n = max(gk)
        roofline = gemm_roofline(w, dom, flops[dom], gbytes[dom], tot / n)
        roofline["traffic"] = traffic_for(dom, w.name)
        hb = hbm_bytes(w, A)
        for name, b in hb.items():
            if name in stages:
                gbs = b / (stages[name]["avg_ms"] / 1e3) / 1e9
                stages[name]["GB/s"] = round(gbs, 1)
                stages[name]["hbm_frac"] = round(gbs / PEAK_HBM_GBS, 3)
        for name in flops:
            if name in stages:
                r = gemm_roofline(w, name, flops[name], gbytes[name], stages[name]["avg_ms"])
                stages[name]["TFLOP/s"] = round(flops[name] / (stages[name]["avg_ms"] / 1e3) / 1e12, 1)
                stages[name]["mfma_frac"] = r["mfma_frac"]
                stages[name]["attainable_frac"] = r["attainable_frac"]
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
        ntok = args.cpu_tokens or CPU_TOKENS.get(w.name, DEFAULT_CPU_TOKENS)
        ntok = min(ntok, w.T)
        log(f"[bench] timing the CPU oracle on {ntok} tokens")
        cpu = cpu_baseline(w, g, ntok)
        log(f"[bench] oracle: {cpu['value']:.2f} tokens/s")

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "median_ms_per_step": round(float(np.median(step_ms)), 4),
        "profiled_ms_per_step": round(prof_ms_step, 4) if prof_ms_step else None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_label(w), "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "E": w.E, "k": w.k, "f": w.f,
                   "act": w.act, "score": w.score, "n_shared": w.n_shared,
                   "capacity": cap, "kept_rows": A, "fp8_fwd": w.fp8, "fp8_dgrad": w.fp8_bwd, "fp8_wgrad": w.fp8_wgrad,
                   "fp8_scale": w.fp8_scale if w.fp8 else None,
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
