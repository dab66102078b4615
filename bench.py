"""Benchmark: one owner-local Muon step over a synthetic matrix set on one MI355X.

Default workload: GPT-2 Large's 144 matrices in bf16 (36 layers x {1280x3840,
1280x1280, 1280x5120, 5120x1280}), 5 Newton-Schulz iterations, mu = 0.95.
A step is one ``muon_step_batched`` call over all matrices (bind, momentum,
norm, 5 x {Gram, polynomial, apply}, fused update), inputs resident in HBM.

Timing follows the blog post's method (appendix ``time_fn``: warmup steps, then
events around the timed steps and the mean): W warmup steps, a synchronize,
HIP events on the launch stream around exactly K steps, a synchronize.  A
second pass of K steps runs with the library's per-launch HIP events on the
same stream to split the step into kernels (the roofline figures).  While the
second pass also reads the clock the GEMM launches ran at, measured inside the
kernels (each workgroup's shader-clock ticks over 100 MHz real-time ticks),
so that the GEMM rate can also be read against the peak at that clock.

The same JSON line also carries, unless switched off: RMNP, column-cut RMNP,
AdamW tails, the MatrixFSDP training configuration, the other configurations
of the benchmark (the float32 single matrix, the Llama-3-8B and 32B-class
owner shares, the ill-conditioned ragged set), the single-matrix size sweep,
and the CPU oracle timed on the whole GPT-2 Large set.

Output: ONE JSON line on stdout (one GPU only: the owner-local step has no
cross-GPU exchange).

``--summarize-profile DIR`` instead reads the CSV output of rocprofv3 runs of
this script (kernel trace, counters) under DIR and prints a per-kernel-class
summary (launches, average duration, MFMA busy, clock, HBM bytes).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Muon step ms + NS TFLOP/s (% bf16 MFMA peak), GPT-2 Large 144-matrix set"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_CLOCK_MHZ = 2400.0       # the engine clock that peak assumes
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
KERNEL_SOURCES = ["matrix_optimizer_step_amd/csrc/ns_gemm_bf16.hip",
                  "matrix_optimizer_step_amd/csrc/common.hpp",
                  "matrix_optimizer_step_amd/csrc/device_util.hpp"]
OTHER_CONFIGS = ("llama3_8b_share_28", "ragged_illcond_64", "qwen32b_share_14")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def ns_alg_flops(shapes, steps):
    """Algorithmic flops of the Newton-Schulz chain with a symmetric Gram:
    per iteration m(m+1)n (upper-triangle X X^T) + m^2(m+1) (upper-triangle
    A A) + 2 m^2 n (B X), m = min side, n = max side."""
    tot = 0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        tot += m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n
    return tot * steps


def prep_alg_bytes(shapes, dtype):
    """Algorithmic HBM bytes of the prep kernel: read G and V, write V, and
    write X0 -- except where X0 would be a copy of V in the same layout (bf16,
    not transposed, both sides multiples of the 256 GEMM tile), which the
    first iteration reads in place."""
    esz = 2 if dtype == "bf16" else 4
    tot = 0
    for r, c in shapes:
        in_place = dtype == "bf16" and r <= c and r % 256 == 0 and c % 256 == 0
        tot += (3 if in_place else 4) * esz * r * c
    return tot


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """Per-launch HBM bytes of the GEMM kernel from committed rocprofv3 --pmc
    counters (profiles/), valid only while the kernel sources are unchanged."""
    path = os.path.join(ROOT, "profiles", f"traffic_ns_gemm_bf16_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(KERNEL_SOURCES):
        return None
    return t.get("bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_steps(fn, steps, warmup, stream):
    """Mean ms of `steps` calls of fn between HIP events on `stream`."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def step_stats(fn, steps, stream):
    """Mean, median and min ms of `steps` calls of fn, each between its own
    HIP events on `stream` (a separate pass from the headline timing)."""
    import statistics
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) for a, b in ev]
    return {"mean": round(sum(t) / len(t), 4), "median": round(statistics.median(t), 4),
            "min": round(min(t), 4)}


def profiled(fn, steps, stream):
    """Per-kernel-class ms per step from the library's per-launch HIP events
    (and the wall ms per step of the pass); bf16 GEMM classes also carry the
    clock (MHz) their launches ran at."""
    import matrix_optimizer_step_amd as mo
    mo.profile_read()
    mo.profile_enable(True)
    mo.profile_read_clock()
    ms = time_steps(fn, steps, 0, stream)
    mo.profile_enable(False)
    prof = mo.profile_read()
    clk = mo.profile_read_clock()
    per = {k: {"ms_per_step": v[0] / steps, "launches_per_step": v[1] / steps}
           for k, v in prof.items() if v[1]}
    for k, mhz in clk.items():
        if k in per:
            per[k]["clock_mhz"] = mhz
    return ms, per


def gemm_clock(per):
    """Time-weighted clock of the GEMM classes (None without clock data)."""
    parts = [(per[k]["ms_per_step"], per[k]["clock_mhz"]) for k in ("gram", "poly", "apply")
             if k in per and "clock_mhz" in per[k]]
    tot = sum(t for t, _ in parts)
    return sum(t * c for t, c in parts) / tot if tot else None


def gemm_rates(per, flops):
    gemm_ms = sum(per[k]["ms_per_step"] for k in ("gram", "poly", "apply") if k in per)
    launches = sum(per[k]["launches_per_step"] for k in ("gram", "poly", "apply") if k in per)
    tflops = flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None
    return gemm_ms, launches, tflops


def cpu_baseline(wl):
    """The oracle (exact float64 mode, unchanged) on the host cores over the
    whole workload, matrix by matrix."""
    import torch
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([p.get("num_threads", 1) for p in info] or [1])
        blas = ",".join(sorted({p.get("internal_api", "?") for p in info}))
    except Exception:  # pragma: no cover
        threads, blas = os.cpu_count() or 1, "?"
    t_total = 0.0
    chunk = 16
    for first in range(0, len(wl.shapes), chunk):
        idx = list(range(first, min(first + chunk, len(wl.shapes))))
        trip = workloads.workload_inputs(wl, idx)
        arrs = [tuple(x.to(torch.float64).numpy() for x in t) for t in trip]
        t0 = time.perf_counter()
        for w, v, g in arrs:
            oracle.muon_step(w, g, v, mu=wl.mu, lr=wl.lr, steps=wl.ns_steps,
                             dtype=wl.dtype, rounding="exact")
        t_total += time.perf_counter() - t0
    return {"value": round(t_total * 1e3, 1), "unit": "ms/step", "cores": int(threads),
            "kind": "oracle",
            "sample": f"all {len(wl.shapes)} matrices of {wl.name}, one step, exact float64 numpy "
                      f"oracle (matrix products through numpy's {blas} float64 GEMM), "
                      f"{threads} threads on {cpu_model()}"}


def vendor_gemm(wl, per, steps, warmup, stream):
    """The same Newton-Schulz products through torch.bmm in bf16 (hipBLASLt),
    as full dense products per distinct shape (X X^T, B B, B X, m <= n), next
    to this library's per-iteration launch times.  Context only: the library
    computes the symmetric Gram and polynomial as upper tiles and fuses the
    polynomial's a I + b A and the Frobenius scale."""
    import torch
    from collections import Counter
    cnt = Counter((min(r, c), max(r, c)) for r, c in wl.shapes)
    tot = {"gram": 0.0, "poly": 0.0, "apply": 0.0}
    for (m, n), c in sorted(cnt.items()):
        X = torch.randn(c, m, n, device="cuda", dtype=torch.bfloat16)
        Xt = X.transpose(1, 2).contiguous()
        B = torch.randn(c, m, m, device="cuda", dtype=torch.bfloat16)
        tot["gram"] += time_steps(lambda: torch.bmm(X, Xt), steps, warmup, stream)
        tot["poly"] += time_steps(lambda: torch.bmm(B, B), steps, warmup, stream)
        tot["apply"] += time_steps(lambda: torch.bmm(B, X), steps, warmup, stream)
        del X, Xt, B
    torch.cuda.empty_cache()
    ours = {k: per[k]["ms_per_step"] / per[k]["launches_per_step"] for k in tot if k in per}
    return {"library": "torch.bmm bf16 (hipBLASLt), full dense products",
            "note": "ours: average launch of the step (the last apply also writes W)",
            "blas_ms_per_iteration": {k: round(v, 4) for k, v in tot.items()},
            "ours_ms_per_iteration": {k: round(v, 4) for k, v in ours.items()},
            "ours_over_blas": {k: round(ours[k] / tot[k], 3) for k in ours}}


def workload_line(name, steps, warmup, stream, with_rmnp=False, with_split=False):
    """Compact line of one more configuration: Muon step ms, NS rate, prep
    bandwidth (and the RMNP step on the same momenta; the step in split
    precision)."""
    import torch
    import matrix_optimizer_step_amd as mo
    import workloads
    wl = workloads.get(name)
    t0 = time.time()
    trip = workloads.workload_inputs(wl)
    W = [t[0].cuda() for t in trip]
    V = [t[1].cuda() for t in trip]
    G = [t[2].cuda() for t in trip]
    del trip
    torch.cuda.synchronize()
    log(f"[bench] {name}: {len(wl.shapes)} matrices resident ({time.time() - t0:.1f} s)")

    def step():
        mo.muon_step_batched(W, G, V, mu=wl.mu, lr=wl.lr, ns_steps=wl.ns_steps)

    ms = time_steps(step, steps, warmup, stream)
    _, per = profiled(step, steps, stream)
    flops = ns_alg_flops(wl.shapes, wl.ns_steps)
    _, _, tflops = gemm_rates(per, flops)
    out = {"workload": name, "dtype": wl.dtype, "matrices": len(wl.shapes),
           "elements": wl.numel, "ms_per_step": round(ms, 4),
           "ns_alg_tflop_per_step": round(flops / 1e12, 4),
           "ns_tflops": round(tflops, 1), "ns_frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
           "gemm_clock_mhz": round(gemm_clock(per) or 0.0, 0),
           "kernels_ms": {k: round(v["ms_per_step"], 4) for k, v in per.items()}}
    if "prep" in per:
        out["prep_GB_s"] = round(prep_alg_bytes(wl.shapes, wl.dtype)
                                 / (per["prep"]["ms_per_step"] * 1e-3) / 1e9, 1)
    log(f"[bench] {name}: muon step {ms:.3f} ms, NS {tflops:.0f} TFLOP/s")
    if with_rmnp:
        rms = time_steps(lambda: mo.rmnp_step_batched(W, G, V, mu=wl.mu, lr=wl.lr),
                         steps, warmup, stream)
        esz = 2 if wl.dtype == "bf16" else 4
        gbs = 5 * esz * wl.numel / (rms * 1e-3) / 1e9
        out["rmnp"] = {"ms_per_step": round(rms, 4), "GB_s": round(gbs, 1),
                       "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                       "muon_over_rmnp": round(ms / rms, 1)}
        log(f"[bench] {name}: rmnp step {rms:.3f} ms ({gbs:.0f} GB/s)")
    if with_split:
        out["split_precision"] = split_line(W, G, V, wl, steps, warmup, stream, ms)
    del W, V, G
    torch.cuda.empty_cache()
    return out


def split_line(W, G, V, wl, steps, warmup, stream, ms_default):
    """The Muon step in split precision (bf16 hi + lo iterates, B X over both
    parts) on the same tensors, beside the default path's ms."""
    import matrix_optimizer_step_amd as mo
    step = lambda: mo.muon_step_batched(W, G, V, mu=wl.mu, lr=wl.lr, ns_steps=wl.ns_steps,
                                        precision="split")
    ms = time_steps(step, steps, warmup, stream)
    _, per = profiled(step, steps, stream)
    gemm_ms = sum(per[k]["ms_per_step"] for k in ("gram", "poly", "apply") if k in per)
    log(f"[bench] {wl.name}: split-precision muon step {ms:.3f} ms ({ms / ms_default:.2f}x)")
    return {"ms_per_step": round(ms, 4), "over_default": round(ms / ms_default, 3),
            "gemm_ms": round(gemm_ms, 4),
            "kernels_ms": {k: round(v["ms_per_step"], 4) for k, v in per.items()}}


def single_f32_line(stream, steps=200, warmup=20, with_oracle=True):
    """The float32 single 256 x 512 matrix: latency-bound (bind, prep,
    finalize, 15 GEMM launches), reported in microseconds per step."""
    import torch
    import matrix_optimizer_step_amd as mo
    import workloads
    wl = workloads.get("single_f32_256x512")
    trip = workloads.workload_inputs(wl)
    W = [t[0].cuda() for t in trip]
    V = [t[1].cuda() for t in trip]
    G = [t[2].cuda() for t in trip]
    ms = time_steps(lambda: mo.muon_step_batched(W, G, V, mu=wl.mu, lr=wl.lr,
                                                 ns_steps=wl.ns_steps), steps, warmup, stream)
    _, per = profiled(lambda: mo.muon_step_batched(W, G, V, mu=wl.mu, lr=wl.lr,
                                                   ns_steps=wl.ns_steps), steps, stream)
    kern_us = sum(v["ms_per_step"] for v in per.values()) * 1e3
    launches = sum(v["launches_per_step"] for v in per.values())
    log(f"[bench] single_f32_256x512: {ms * 1e3:.1f} us/step")
    out = {"workload": wl.name, "dtype": "f32", "us_per_step": round(ms * 1e3, 2),
           "kernel_us_per_step": round(kern_us, 2), "launches_per_step": launches,
           "steps": steps}
    if with_oracle:
        # the oracle (exact float64) on the same matrix, one step at a time
        import oracle
        w, v, g = (x.to(torch.float64).numpy() for x in trip[0])
        reps = 20
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.muon_step(w, g, v.copy(), mu=wl.mu, lr=wl.lr, steps=wl.ns_steps,
                             dtype=wl.dtype, rounding="exact")
        out["cpu_oracle_us_per_step"] = round((time.perf_counter() - t0) / reps * 1e6, 1)
    return out


def square_sweep(steps, warmup, stream):
    """One s x s bf16 matrix per size (the blog post's single-matrix size sweep,
    without the gather that its distributed setting adds): the whole Muon step,
    Newton-Schulz alone, and the RMNP step, each timed like the main bench."""
    import torch
    import matrix_optimizer_step_amd as mo
    import workloads
    rows = []
    for sz in workloads.SWEEP_SIZES:
        wl = workloads.square_sweep(sz)
        trip = workloads.workload_inputs(wl)
        W = [trip[0][0].cuda()]
        V = [trip[0][1].cuda()]
        G = [trip[0][2].cuda()]
        O = [torch.empty(sz, sz, dtype=torch.bfloat16, device="cuda")]
        muon = time_steps(lambda: mo.muon_step_batched(W, G, V, mu=0.95, lr=0.02, ns_steps=5),
                          steps, warmup, stream)
        ns = time_steps(lambda: mo.ns_orthogonalize_batched(V, out_dtype=torch.bfloat16, outs=O),
                        steps, warmup, stream)
        rmnp = time_steps(lambda: mo.rmnp_step_batched(W, G, V, mu=0.95, lr=0.02),
                          steps, warmup, stream)
        fl = ns_alg_flops([(sz, sz)], 5)
        rows.append({"s": sz, "muon_step_ms": round(muon, 4), "ns_ms": round(ns, 4),
                     "rmnp_step_ms": round(rmnp, 4), "muon_over_rmnp": round(muon / rmnp, 1),
                     "ns_tflops": round(fl / (ns * 1e-3) / 1e12, 1),
                     "rmnp_GB_s": round(10 * sz * sz / (rmnp * 1e-3) / 1e9, 1)})
        log(f"[bench] sweep {sz}x{sz}: muon {muon:.3f} ms, NS {ns:.3f} ms, rmnp {rmnp:.3f} ms")
        del W, V, G, O
    return rows


# ------------------------------------------------------------ profile summary
GEMM_CLASS = {"0": "gram", "1": "poly"}


def kernel_class(name):
    """Kernel class of a rocprofv3 kernel name (the library's kernels only)."""
    if "ns_apply_persist_kernel" in name:
        return "apply"
    if "prep_t_kernel" in name:   # the transposed bf16 matrices' prep launch
        return "prep"
    m = re.search(r"ns_gemm_bf16_kernel<(\d+), (\d+), \d+(?:, (?:true|false))?>", name)
    if m:
        st, out = m.group(1), m.group(2)
        if st in GEMM_CLASS:
            return GEMM_CLASS[st]
        return "apply" if out == "0" else "apply_final"
    for k in ("prep_kernel", "finalize_kernel", "scale_out_kernel", "rmnp_kernel",
              "colcut_partial_kernel", "colcut_apply_kernel", "adamw_kernel", "bind_kernel",
              "ns_gemm_f32_kernel"):
        if k in name:
            return k.replace("_kernel", "")
    if "copy" in name.lower() or "Copy" in name:
        return "copy"
    return None


def summarize_profile(directory, flops_per_step=None, steps=None):
    """Per-class table from rocprofv3 CSVs under `directory`: kernel trace
    (durations) and counter collection (MFMA busy, clock, FETCH/WRITE sizes)."""
    rows = {}
    for path in glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                cls = kernel_class(r.get("Kernel_Name", ""))
                if not cls:
                    continue
                d = rows.setdefault(cls, {"n": 0, "ns": 0.0})
                d["n"] += 1
                d["ns"] += float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    counters = {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                cls = kernel_class(r.get("Kernel_Name", ""))
                if not cls:
                    continue
                c = counters.setdefault(cls, {}).setdefault(r["Counter_Name"], [])
                c.append(float(r["Counter_Value"]))
    out = {}
    for cls in sorted(set(rows) | set(counters)):
        d = {}
        if cls in rows:
            d["launches"] = rows[cls]["n"]
            d["avg_us"] = rows[cls]["ns"] / rows[cls]["n"] / 1e3
        for name, vals in counters.get(cls, {}).items():
            d[name + "_avg"] = sum(vals) / len(vals)
            d[name + "_max"] = max(vals)
        if "avg_us" in d and "GRBM_GUI_ACTIVE_avg" in d:
            # GRBM_GUI_ACTIVE counts GPU cycles summed over the 8 XCDs
            ghz = d["GRBM_GUI_ACTIVE_avg"] / 8 / (d["avg_us"] * 1e3)
            d["clock_GHz"] = ghz
            if "SQ_VALU_MFMA_BUSY_CYCLES_avg" in d:
                # MFMA busy cycles summed over the 1024 SIMDs (256 CUs x 4)
                d["mfma_busy"] = d["SQ_VALU_MFMA_BUSY_CYCLES_avg"] / 1024 / (
                    d["GRBM_GUI_ACTIVE_avg"] / 8)
        out[cls] = d
    return out


def zero_data_line(wl, W, G, V, steps, warmup, stream):
    """The step on the set's own G, V and on all-zero G, V: the same launches,
    tables and instructions (the iterates are then zero throughout), so any
    difference in time comes from what the data does to the clock."""
    import torch
    import matrix_optimizer_step_amd as mo
    out = {"diagnostic": "same launches on Gaussian and on all-zero G, V", "workload": wl.name,
           "steps": steps, "warmup": warmup}
    zeros = ([torch.zeros_like(g) for g in G], [torch.zeros_like(v) for v in V])
    for label, (g_, v_) in (("gaussian", (G, V)), ("zero", zeros)):
        def step():
            mo.muon_step_batched(W, g_, v_, mu=wl.mu, lr=wl.lr, ns_steps=wl.ns_steps)
        ms = time_steps(step, steps, warmup, stream)
        _, per = profiled(step, steps, stream)
        _, _, tf = gemm_rates(per, ns_alg_flops(wl.shapes, wl.ns_steps))
        out[label] = {
            "ms_per_step": round(ms, 4),
            "gemm_clock_mhz": round(gemm_clock(per) or 0.0),
            "ns_frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4) if tf else None,
            "us_per_launch": {k: round(v["ms_per_step"] * 1e3 / v["launches_per_step"], 1)
                              for k, v in per.items() if k in ("gram", "poly", "apply")},
            "clock_mhz": {k: round(v.get("clock_mhz", 0.0)) for k, v in per.items()
                          if k in ("gram", "poly", "apply")},
        }
    return out


def card_power_files():
    """The GPU's hwmon power readings (microwatts), where the box exposes them."""
    import glob
    out = []
    for f in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input")):
        try:
            int(open(f).read())
            out.append(f)
        except (OSError, ValueError):
            pass
    return out


def mfma_probe_line(stream, launches=40, iters=3000, workgroups=2048, cases=None):
    """Diagnostic: the library's MFMA rate probe (matopt_mfma_probe) for both
    MFMA forms, operands in registers or read from LDS each step, on Gaussian
    and on all-zero bf16 data: TFLOP/s, the clock the loop ran at (shader over
    real-time ticks), MFMA utilisation at that clock, and the card's power
    reading sampled every 20 ms while the timed launches ran."""
    import threading
    import torch
    import matrix_optimizer_step_amd as mo
    g = torch.Generator().manual_seed(5)
    data = {"gaussian": torch.randn(49152, generator=g).to(torch.bfloat16).cuda(),
            "zero": torch.zeros(49152, dtype=torch.bfloat16, device="cuda")}
    out = torch.empty(workgroups * 512, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    pw_files = card_power_files()
    flops = workgroups * 8 * iters * 524288
    cases = cases or [(32, False, "gaussian"), (16, False, "gaussian"), (32, True, "gaussian"),
                      (16, True, "gaussian"), (32, True, "zero"), (16, True, "zero")]
    res = []
    for form, lds, dname in cases:
        for _ in range(3):
            mo.mfma_probe(form, lds, data[dname], out, clk, iters, workgroups, stream)
        torch.cuda.synchronize()
        clk.zero_()
        samples, stop = [], threading.Event()

        def sample():
            while not stop.is_set():
                for f in pw_files:
                    try:
                        samples.append(int(open(f).read()) / 1e6)
                    except (OSError, ValueError):
                        pass
                time.sleep(0.02)
        th = threading.Thread(target=sample)
        th.start()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            mo.mfma_probe(form, lds, data[dname], out, clk, iters, workgroups, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        stop.set()
        th.join()
        ms = e0.elapsed_time(e1) / launches
        c = clk.cpu().tolist()
        mhz = 100.0 * c[0] / c[1] if c[1] else 0.0
        tf = flops / (ms * 1e-3) / 1e12
        half = samples[len(samples) // 2:]   # the ramp-up excluded
        res.append({"mfma": {32: "32x32x16", 16: "16x16x32"}[form],
                    "operands": "LDS, read one step ahead" if lds else "registers",
                    "data": dname, "ms_per_launch": round(ms, 3), "tflops": round(tf, 1),
                    "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "clock_mhz": round(mhz),
                    "busy_at_clock": round(tf / PEAK_BF16_TFLOPS * 2400.0 / mhz, 3) if mhz else None,
                    "power_w_mean": round(sum(half) / len(half), 1) if half else None,
                    "power_w_max": round(max(half), 1) if half else None})
    return {"diagnostic": "MFMA rate probe (matopt_mfma_probe): both MFMA forms on register or "
                          "LDS operands, Gaussian and all-zero bf16 data",
            "workgroups": workgroups, "iters": iters, "launches": launches,
            "flop_per_launch": flops, "power_source": pw_files or None, "cases": res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt2_large_144")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rmnp", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configurations (float32 single matrix, Llama-3-8B "
                         "share, ill-conditioned set, 32B-class share)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the single-matrix sweep")
    ap.add_argument("--step-only", action="store_true",
                    help="time the Muon step of --workload only (no RMNP, column-cut RMNP, "
                         "AdamW, training-configuration, other configurations or sweep "
                         "lines), e.g. for a profiler run")
    ap.add_argument("--sweep", action="store_true",
                    help="only the single-matrix sweep (s = 1024..8192), as its own JSON line")
    ap.add_argument("--zero-data", action="store_true",
                    help="diagnostic only: the same step on the set's Gaussian G, V and on "
                         "all-zero G, V (identical launches and instructions, no data toggling), "
                         "one JSON line with both times and the GEMM clocks; no headline line")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="diagnostic only: the library's MFMA rate probe for both MFMA forms "
                         "(registers / LDS operands, Gaussian / zero data) with the card's power "
                         "reading, one JSON line; no headline line")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (float32), the "
                         "known-size kernel that scales rocprofv3 FETCH_SIZE/WRITE_SIZE readings")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="print a per-kernel-class summary of the rocprofv3 CSV output under DIR "
                         "and exit (no GPU use)")
    args = ap.parse_args()
    if args.summarize_profile:
        print(json.dumps(summarize_profile(args.summarize_profile), indent=1))
        return
    if args.step_only:
        args.no_rmnp = args.no_configs = args.no_sweep = True

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): the owner-local Muon step has no cross-GPU exchange; each GPU would "
              f"run this same step on the matrices it owns.", file=sys.stderr)
        sys.exit(2)

    import torch
    import matrix_optimizer_step_amd as mo
    import workloads

    mo.lib()
    stream = torch.cuda.current_stream()
    if args.mfma_probe:
        print(json.dumps(mfma_probe_line(stream)), flush=True)
        return
    if args.sweep:
        print(json.dumps({"metric": "single s x s bf16 matrix: Muon step vs RMNP step (ms)",
                          "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "dtype": "bf16", "data": "synthetic (seeded numpy Gaussians)",
                          "config": {"workload": "square_sweep",
                                     "sizes": list(workloads.SWEEP_SIZES), "ns_steps": 5},
                          "sweep": square_sweep(args.steps, args.warmup, stream)}), flush=True)
        return
    wl = workloads.get(args.workload)
    log(f"[bench] workload {wl.name}: {len(wl.shapes)} matrices, {wl.numel / 1e6:.1f}M elements")
    t0 = time.time()
    trip = workloads.workload_inputs(wl)
    W = [t[0].cuda() for t in trip]
    V = [t[1].cuda() for t in trip]
    G = [t[2].cuda() for t in trip]
    del trip
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM ({time.time() - t0:.1f} s)")
    if args.calib_copy_mib:
        n = args.calib_copy_mib * 2 ** 20 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done")

    if args.zero_data:
        print(json.dumps(zero_data_line(wl, W, G, V, args.steps, args.warmup, stream)), flush=True)
        return

    def step():
        mo.muon_step_batched(W, G, V, mu=wl.mu, lr=wl.lr, ns_steps=wl.ns_steps)

    ms = time_steps(step, args.steps, args.warmup, stream)
    log(f"[bench] muon step {ms:.3f} ms")
    per_step = step_stats(step, args.steps, stream)

    # second pass: per-launch HIP events inside the library, same stream
    ms_prof, per = profiled(step, args.steps, stream)
    clock = gemm_clock(per)
    flops = ns_alg_flops(wl.shapes, wl.ns_steps)
    gemm_ms, gemm_launches, ns_tflops = gemm_rates(per, flops)
    numel = wl.numel
    esz = 2 if wl.dtype == "bf16" else 4
    prep_gbs = None
    prep_bytes = prep_alg_bytes(wl.shapes, wl.dtype)
    if "prep" in per:
        prep_gbs = prep_bytes / (per["prep"]["ms_per_step"] * 1e-3) / 1e9
    traffic = load_traffic(wl.name)
    roofline = {
        "kernel": "ns_gemm_bf16_kernel and ns_apply_persist_kernel (Gram, polynomial and apply launches)",
        "bound": "mfma",
        "achieved": round(ns_tflops, 1) if ns_tflops else None,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(ns_tflops / PEAK_BF16_TFLOPS, 4) if ns_tflops else None,
        "traffic": traffic,
        "flop_per_launch": round(flops / gemm_launches) if gemm_launches else None,
        "avg_launch_ms": round(gemm_ms / gemm_launches, 5) if gemm_launches else None,
    }
    if clock and ns_tflops:
        peak_obs = PEAK_BF16_TFLOPS * clock / PEAK_CLOCK_MHZ
        roofline["observed_clock_mhz"] = round(clock, 0)
        roofline["observed_clock_source"] = (
            "measured in the GEMM kernels during the profiled pass: shader-clock ticks over "
            "100 MHz real-time ticks per workgroup, time-weighted over Gram, polynomial, apply")
        roofline["peak_at_observed_clock"] = round(peak_obs, 1)
        roofline["frac_at_observed_clock"] = round(ns_tflops / peak_obs, 4)
    if ns_tflops and not args.step_only:
        # the rate MFMAs fed from LDS alone sustain on this part with Gaussian
        # bf16 operands (no DMA, no epilogue): a bound for any schedule of the
        # chain on the same data; about a second of launches, so that the
        # clock has settled as it has in the chain's timed steps
        probe = mfma_probe_line(stream, launches=60, iters=3000, cases=[(16, True, "gaussian")])
        c = probe["cases"][0]
        roofline["mfma_lds_ceiling"] = {
            "tflops": c["tflops"], "frac_bf16_peak": c["frac_bf16_peak"],
            "clock_mhz": c["clock_mhz"],
            "source": "matopt_mfma_probe in this run: 16x16x32 bf16 MFMAs on fragments read "
                      "from LDS one step ahead, Gaussian operands, no DMA, no epilogue"}
        roofline["frac_of_mfma_lds_ceiling"] = round(ns_tflops / c["tflops"], 4)

    result = {
        "metric": METRIC,
        "value": round(ms, 4),
        "unit": "ms/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded numpy Gaussians, shapes of the named matrix set)",
        "config": {"workload": wl.name, "matrices": len(wl.shapes), "elements": numel,
                   "ns_steps": wl.ns_steps, "mu": wl.mu, "lr": wl.lr,
                   "ns_coeffs": list(mo.NS_COEFFS), "eps": 1e-7},
        "ns_tflops": round(ns_tflops, 1) if ns_tflops else None,
        "ns_pct_bf16_peak": round(100 * ns_tflops / PEAK_BF16_TFLOPS, 2) if ns_tflops else None,
        "ns_alg_tflop_per_step": round(flops / 1e12, 4),
        "roofline": roofline,
        "kernels": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in per.items()},
        "ms_per_step_profiled": round(ms_prof, 4),
        "ms_per_step_each": per_step,
        "hbm_kernels": {
            "prep": {"bytes_per_elem": round(prep_bytes / numel, 3),
                     "GB_s": round(prep_gbs, 1) if prep_gbs else None,
                     "frac_hbm": round(prep_gbs / PEAK_HBM_GBS, 4) if prep_gbs else None},
        },
    }

    if not args.no_rmnp:
        result["vendor_gemm"] = vendor_gemm(wl, per, args.steps, args.warmup, stream)
        log(f"[bench] vendor GEMM reference: {result['vendor_gemm']['ours_over_blas']}")
        rms = time_steps(lambda: mo.rmnp_step_batched(W, G, V, mu=wl.mu, lr=wl.lr),
                         args.steps, args.warmup, stream)
        gbs = 5 * esz * numel / (rms * 1e-3) / 1e9
        result["rmnp"] = {"ms_per_step": round(rms, 4), "bytes_per_elem": 5 * esz,
                          "GB_s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                          "muon_over_rmnp": round(ms / rms, 1)}
        log(f"[bench] rmnp step {rms:.3f} ms ({gbs:.0f} GB/s)")

        # Column-cut RMNP, both local halves on whole-width slices (one rank:
        # the sum over ranks between them is the identity)
        rowsq = torch.empty(sum(r for r, _ in wl.shapes), dtype=torch.float32, device="cuda")

        def colcut():
            mo.rmnp_colcut_partial_batched(G, V, rowsq=rowsq, mu=wl.mu)
            mo.rmnp_colcut_apply_batched(W, V, rowsq, lr=wl.lr)

        cms = time_steps(colcut, args.steps, args.warmup, stream)
        _, cp = profiled(colcut, args.steps, stream)
        cgbs = 12 * esz / 2 * numel / (cms * 1e-3) / 1e9
        result["rmnp_colcut"] = {
            "ms_per_step": round(cms, 4), "bytes_per_elem": 6 * esz, "GB_s": round(cgbs, 1),
            "frac_hbm": round(cgbs / PEAK_HBM_GBS, 4),
            "partial_ms": round(cp["colcut_partial"]["ms_per_step"], 4),
            "apply_ms": round(cp["colcut_apply"]["ms_per_step"], 4)}
        log(f"[bench] column-cut rmnp {cms:.3f} ms ({cgbs:.0f} GB/s)")

        # AdamW on the non-2D tail: GPT-2 Large's LayerNorm weights and biases
        # and its linear biases (36 layers x {1280 x 6, 3840, 5120} + the final
        # LayerNorm's 2 x 1280: 290 tensors, 601,600 elements; bf16 parameters,
        # float32 moments) as 290 tensors and as one flat tensor (the tail kept
        # as one owner role), then a 64M-element tail for the HBM rate.
        # kernel_us is the library's own per-launch HIP-event time; wall_us also
        # holds the Python marshalling of the tensor list.
        tail = [1280, 1280, 3840, 1280, 1280, 1280, 5120, 1280] * 36 + [1280, 1280]
        result["adamw"] = {}
        for name, lens in (("gpt2_large_tail_290", tail), ("gpt2_large_tail_flat", [sum(tail)]),
                           ("tail_64M", [1 << 24] * 4)):
            tp = [torch.randn(n, device="cuda").bfloat16() for n in lens]
            tg = [(torch.randn(n, device="cuda") * 0.1).bfloat16() for n in lens]
            tm = [torch.zeros(n, device="cuda") for n in lens]
            tv = [torch.zeros(n, device="cuda") for n in lens]
            st = [0]

            def adamw():
                st[0] += 1
                mo.adamw_step_batched(tp, tg, tm, tv, st[0])

            wall = time_steps(adamw, args.steps, args.warmup, stream)
            _, ap_ = profiled(adamw, args.steps, stream)
            kms = ap_["adamw"]["ms_per_step"]
            nel = sum(lens)
            agbs = 22 * nel / (kms * 1e-3) / 1e9
            result["adamw"][name] = {"tensors": len(lens), "elements": nel,
                                     "kernel_us": round(kms * 1e3, 2),
                                     "wall_us": round(wall * 1e3, 2), "bytes_per_elem": 22,
                                     "GB_s": round(agbs, 1), "frac_hbm": round(agbs / PEAK_HBM_GBS, 4)}
            log(f"[bench] adamw {name}: kernel {kms * 1e3:.1f} us ({agbs:.0f} GB/s), "
                f"wall {wall * 1e3:.1f} us")
            del tp, tg, tm, tv

        # MatrixFSDP's training configuration (section 5.1) on the same
        # matrices: momentum 0.5, 2 Newton-Schulz steps, decoupled weight decay
        # 1e-2, lr 1e-3
        wms = time_steps(lambda: mo.muon_step_batched_wd(W, G, V, mu=0.5, lr=1e-3, wd=1e-2,
                                                         ns_steps=2),
                         args.steps, args.warmup, stream)
        result["split_precision"] = split_line(W, G, V, wl, args.steps, args.warmup, stream, ms)
        result["training_config"] = {"ms_per_step": round(wms, 4), "mu": 0.5, "lr": 1e-3,
                                     "wd": 1e-2, "ns_steps": 2,
                                     "ns_alg_tflop_per_step": round(ns_alg_flops(wl.shapes, 2) / 1e12, 4)}
        log(f"[bench] training-config muon step {wms:.3f} ms")

    del W, V, G
    torch.cuda.empty_cache()
    if not args.no_configs:
        result["configs"] = {"single_f32_256x512": single_f32_line(stream)}
        for name in OTHER_CONFIGS:
            result["configs"][name] = workload_line(name, args.steps, args.warmup, stream,
                                                    with_rmnp=name == "qwen32b_share_14",
                                                    with_split=name == "ragged_illcond_64")
    if not args.no_sweep:
        result["sweep"] = square_sweep(args.steps, args.warmup, stream)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on the whole set ...")
        result["cpu_baseline"] = cpu_baseline(wl)
        log(f"[bench] CPU oracle {result['cpu_baseline']['value'] / 1e3:.1f} s/step")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
