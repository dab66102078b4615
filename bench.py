"""Benchmark: one owner-local Muon step over a synthetic matrix set on one MI355X.

Default workload: GPT-2 Large's 144 matrices in bf16 (36 layers x {1280x3840,
1280x1280, 1280x5120, 5120x1280}), 5 Newton-Schulz iterations, mu = 0.95.
A step is one ``muon_step_batched`` call over all matrices (momentum, norm,
5 x {Gram, polynomial, apply}, fused update), inputs resident in HBM.

Timing follows the blog post's method (appendix ``time_fn``: warmup steps, then
events around the timed steps and the mean): W warmup steps, a synchronize,
HIP events on the launch stream around exactly K steps, a synchronize.  A
second pass of K steps runs with the library's per-launch HIP events on the
same stream to split the step into kernels (the roofline figures).

Output: ONE JSON line on stdout (rank 0; this build runs on one GPU only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Muon step ms + NS TFLOP/s (% bf16 MFMA peak), GPT-2 Large 144-matrix set"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
KERNEL_SOURCES = ["matrix_optimizer_step_amd/csrc/ns_gemm_bf16.hip",
                  "matrix_optimizer_step_amd/csrc/common.hpp",
                  "matrix_optimizer_step_amd/csrc/device_util.hpp"]


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


def cpu_baseline(wl, budget_s=15.0):
    """The oracle (exact float64 mode, unchanged) on the host cores, on the first
    layers of the same workload until ~budget_s of work, extrapolated by matrix
    count to a whole step."""
    import torch
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    per_layer = 4 if wl.name == "gpt2_large_144" else 1
    done = 0
    t_total = 0.0
    while done < len(wl.shapes) and t_total < budget_s:
        idx = list(range(done, min(done + per_layer, len(wl.shapes))))
        trip = workloads.workload_inputs(wl, idx)
        arrs = [tuple(x.to(torch.float64).numpy() for x in t) for t in trip]
        t0 = time.perf_counter()
        for w, v, g in arrs:
            oracle.muon_step(w, g, v, mu=wl.mu, lr=wl.lr, steps=wl.ns_steps,
                             dtype=wl.dtype, rounding="exact")
        t_total += time.perf_counter() - t0
        done += len(idx)
    frac = sum(r * c for r, c in wl.shapes[:done]) / wl.numel
    flop_frac = ns_alg_flops(wl.shapes[:done], 1) / ns_alg_flops(wl.shapes, 1)
    ms = t_total / flop_frac * 1e3
    return {"value": round(ms, 1), "unit": "ms/step (extrapolated)",
            "cores": int(threads), "kind": "oracle",
            "sample": f"first {done} of {len(wl.shapes)} matrices ({frac:.1%} of elements, "
                      f"{flop_frac:.1%} of NS flops), exact float64 numpy oracle, "
                      f"{t_total:.1f} s measured, scaled by NS flop share"}


def square_sweep(args):
    """One s x s bf16 matrix per size (the blog post's single-matrix size sweep,
    without the gather that its distributed setting adds): the whole Muon step,
    Newton-Schulz alone, and the RMNP step, each timed like the main bench."""
    import torch
    import matrix_optimizer_step_amd as mo
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    rows = []
    g = torch.Generator(device="cuda")
    g.manual_seed(1337)
    for sz in (1024, 2048, 4096, 8192):
        W = [(torch.randn(sz, sz, device="cuda", generator=g) * 0.02).bfloat16()]
        V = [(torch.randn(sz, sz, device="cuda", generator=g) * 1e-3).bfloat16()]
        G = [(torch.randn(sz, sz, device="cuda", generator=g) * 1e-3).bfloat16()]
        O = [torch.empty(sz, sz, dtype=torch.bfloat16, device="cuda")]
        muon = timed(lambda: mo.muon_step_batched(W, G, V, mu=0.95, lr=0.02, ns_steps=5))
        ns = timed(lambda: mo.ns_orthogonalize_batched(V, out_dtype=torch.bfloat16, outs=O))
        rmnp = timed(lambda: mo.rmnp_step_batched(W, G, V, mu=0.95, lr=0.02))
        fl = ns_alg_flops([(sz, sz)], 5)
        rows.append({"s": sz, "muon_step_ms": round(muon, 4), "ns_ms": round(ns, 4),
                     "rmnp_step_ms": round(rmnp, 4), "muon_over_rmnp": round(muon / rmnp, 1),
                     "ns_tflops": round(fl / (ns * 1e-3) / 1e12, 1),
                     "rmnp_GB_s": round(10 * sz * sz / (rmnp * 1e-3) / 1e9, 1)})
        log(f"[sweep] {sz}x{sz}: muon {muon:.3f} ms, NS {ns:.3f} ms, rmnp {rmnp:.3f} ms")
        del W, V, G, O
    return {"metric": "single s x s bf16 matrix: Muon step vs RMNP step (ms)", "unit": "ms",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "dtype": "bf16",
            "data": "synthetic (torch.randn, W 0.02, V and G 1e-3)",
            "config": {"workload": "square_sweep", "sizes": [1024, 2048, 4096, 8192],
                       "ns_steps": 5}, "sweep": rows}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt2_large_144")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rmnp", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="time the Muon step only (no RMNP, column-cut RMNP, AdamW or "
                         "training-configuration lines), e.g. for a profiler run")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step benchmark: one s x s bf16 matrix for s in "
                         "1024..8192, Muon step vs Newton-Schulz alone vs RMNP step")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (float32), the "
                         "known-size kernel that scales rocprofv3 FETCH_SIZE/WRITE_SIZE readings")
    args = ap.parse_args()
    if args.step_only:
        args.no_rmnp = True

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
    if args.sweep:
        print(json.dumps(square_sweep(args)), flush=True)
        return
    wl = workloads.get(args.workload)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    log(f"[bench] workload {wl.name}: {len(wl.shapes)} matrices, {wl.numel / 1e6:.1f}M elements")
    t0 = time.time()
    trip = workloads.workload_inputs(wl)
    W = [t[0].cuda() for t in trip]
    V = [t[1].cuda() for t in trip]
    G = [t[2].cuda() for t in trip]
    del trip
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM ({time.time() - t0:.1f} s)")
    stream = torch.cuda.current_stream()
    if args.calib_copy_mib:
        n = args.calib_copy_mib * 2 ** 20 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done")

    def step():
        mo.muon_step_batched(W, G, V, mu=wl.mu, lr=wl.lr, ns_steps=wl.ns_steps)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] muon step {ms:.3f} ms")

    # second pass: per-launch HIP events inside the library, same stream
    mo.profile_read()
    mo.profile_enable(True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_prof = e0.elapsed_time(e1) / args.steps
    mo.profile_enable(False)
    prof = mo.profile_read()
    per = {k: {"ms_per_step": v[0] / args.steps, "launches_per_step": v[1] / args.steps}
           for k, v in prof.items() if v[1]}

    flops = ns_alg_flops(wl.shapes, wl.ns_steps)
    gemm_ms = sum(per[k]["ms_per_step"] for k in ("gram", "poly", "apply") if k in per)
    gemm_launches = sum(per[k]["launches_per_step"] for k in ("gram", "poly", "apply") if k in per)
    ns_tflops = flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None
    numel = wl.numel
    esz = 2 if wl.dtype == "bf16" else 4
    prep_gbs = None
    prep_bytes = prep_alg_bytes(wl.shapes, wl.dtype)
    if "prep" in per:
        prep_gbs = prep_bytes / (per["prep"]["ms_per_step"] * 1e-3) / 1e9
    traffic = load_traffic(wl.name)

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
        "roofline": {
            "kernel": "ns_gemm_bf16_kernel (Gram, polynomial and apply launches)",
            "bound": "mfma",
            "achieved": round(ns_tflops, 1) if ns_tflops else None,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(ns_tflops / PEAK_BF16_TFLOPS, 4) if ns_tflops else None,
            "traffic": traffic,
            "flop_per_launch": round(flops / gemm_launches) if gemm_launches else None,
            "avg_launch_ms": round(gemm_ms / gemm_launches, 5) if gemm_launches else None,
        },
        "kernels": {k: {"ms_per_step": round(v["ms_per_step"], 4),
                        "launches_per_step": v["launches_per_step"]} for k, v in per.items()},
        "ms_per_step_profiled": round(ms_prof, 4),
        "hbm_kernels": {
            "prep": {"bytes_per_elem": round(prep_bytes / numel, 3),
                     "GB_s": round(prep_gbs, 1) if prep_gbs else None,
                     "frac_hbm": round(prep_gbs / PEAK_HBM_GBS, 4) if prep_gbs else None},
        },
    }

    if not args.no_rmnp:
        for _ in range(args.warmup):
            mo.rmnp_step_batched(W, G, V, mu=wl.mu, lr=wl.lr)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            mo.rmnp_step_batched(W, G, V, mu=wl.mu, lr=wl.lr)
        e1.record(stream)
        torch.cuda.synchronize()
        rms = e0.elapsed_time(e1) / args.steps
        gbs = 5 * esz * numel / (rms * 1e-3) / 1e9
        result["rmnp"] = {"ms_per_step": round(rms, 4), "bytes_per_elem": 5 * esz,
                          "GB_s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                          "muon_over_rmnp": round(ms / rms, 1)}
        log(f"[bench] rmnp step {rms:.3f} ms ({gbs:.0f} GB/s)")

    # Column-cut RMNP, both local halves on whole-width slices (one rank: the
    # sum over ranks between them is the identity)
    if not args.no_rmnp:
        rowsq = torch.empty(sum(r for r, _ in wl.shapes), dtype=torch.float32, device="cuda")

        def colcut():
            mo.rmnp_colcut_partial_batched(G, V, rowsq=rowsq, mu=wl.mu)
            mo.rmnp_colcut_apply_batched(W, V, rowsq, lr=wl.lr)

        for _ in range(args.warmup):
            colcut()
        torch.cuda.synchronize()
        mo.profile_read()
        mo.profile_enable(True)
        e0.record(stream)
        for _ in range(args.steps):
            colcut()
        e1.record(stream)
        torch.cuda.synchronize()
        mo.profile_enable(False)
        cms = e0.elapsed_time(e1) / args.steps
        cp = mo.profile_read()
        cgbs = 12 * esz / 2 * numel / (cms * 1e-3) / 1e9
        result["rmnp_colcut"] = {
            "ms_per_step": round(cms, 4), "bytes_per_elem": 6 * esz, "GB_s": round(cgbs, 1),
            "frac_hbm": round(cgbs / PEAK_HBM_GBS, 4),
            "partial_ms": round(cp["colcut_partial"][0] / args.steps, 4),
            "apply_ms": round(cp["colcut_apply"][0] / args.steps, 4)}
        log(f"[bench] column-cut rmnp {cms:.3f} ms ({cgbs:.0f} GB/s)")

    # AdamW on the non-2D tail: GPT-2 Large's LayerNorm weights and biases and
    # its linear biases (36 layers x {1280 x 6, 3840, 5120} + the final
    # LayerNorm's 2 x 1280: 290 tensors, 601,600 elements; bf16 parameters,
    # float32 moments) as 290 tensors and as one flat tensor (the tail kept as
    # one owner role), then a 64M-element tail for the HBM rate.  kernel_us is
    # the library's own per-launch HIP-event time; wall_us also holds the
    # Python marshalling of the tensor list.
    if not args.no_rmnp:
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

            for _ in range(args.warmup):
                adamw()
            torch.cuda.synchronize()
            mo.profile_read()
            mo.profile_enable(True)
            e0.record(stream)
            for _ in range(args.steps):
                adamw()
            e1.record(stream)
            torch.cuda.synchronize()
            mo.profile_enable(False)
            wall = e0.elapsed_time(e1) / args.steps
            kms = mo.profile_read()["adamw"][0] / args.steps
            nel = sum(lens)
            agbs = 22 * nel / (kms * 1e-3) / 1e9
            result["adamw"][name] = {"tensors": len(lens), "elements": nel,
                                     "kernel_us": round(kms * 1e3, 2),
                                     "wall_us": round(wall * 1e3, 2), "bytes_per_elem": 22,
                                     "GB_s": round(agbs, 1), "frac_hbm": round(agbs / PEAK_HBM_GBS, 4)}
            log(f"[bench] adamw {name}: kernel {kms * 1e3:.1f} us ({agbs:.0f} GB/s), "
                f"wall {wall * 1e3:.1f} us")
            del tp, tg, tm, tv

    # MatrixFSDP's training configuration (section 5.1) on the same matrices:
    # momentum 0.5, 2 Newton-Schulz steps, decoupled weight decay 1e-2, lr 1e-3
    if args.step_only:
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
        print(json.dumps(result), flush=True)
        return

    def step_wd():
        mo.muon_step_batched_wd(W, G, V, mu=0.5, lr=1e-3, wd=1e-2, ns_steps=2)

    for _ in range(args.warmup):
        step_wd()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step_wd()
    e1.record(stream)
    torch.cuda.synchronize()
    wms = e0.elapsed_time(e1) / args.steps
    result["training_config"] = {"ms_per_step": round(wms, 4), "mu": 0.5, "lr": 1e-3,
                                 "wd": 1e-2, "ns_steps": 2,
                                 "ns_alg_tflop_per_step": round(ns_alg_flops(wl.shapes, 2) / 1e12, 4)}
    log(f"[bench] training-config muon step {wms:.3f} ms")

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
