"""Benchmark: ExTernD decomposition throughput on one MI355X.

One step = one full decomposition (the whole hot path) of the workload's synthetic matrix,
already resident in HBM.  Default workload: the attention-projection case, A 2560 x 2560
(Student-t nu=4 at std 0.02, 8 outlier columns x20), mu = 3 (k = 7680), tau = 0, 4 ALS
iterations, sequential deflation.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
    python bench.py --probe            # sustained read / copy bandwidth at 26 MB, 100 MB, 1 GB
    python bench.py --oracle-timings   # the oracle on one and on all host cores (small workloads)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources of each path's kernels: a counter figure stays valid while these files are unchanged.
KERNEL_SOURCES = {"seq": ("seq.hip", "select.hpp", "common.hpp"),
                  "block": ("block.hip", "select.hpp", "common.hpp")}


def source_digest(path="seq"):
    """sha256 over the sources of one path's kernels (seq or block)."""
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[path]:
        h.update(name.encode())
        with open(os.path.join(here, "expanded_rank_matrix_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's reading), or None when they were taken
    on other kernel sources."""
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_digest") != source_digest(t.get("path", "seq")):
        return None
    return float(t["traffic_bytes_per_launch"])


def copy_probe(megabytes):
    """A plain device copy of known size, timed by the counter runs to scale FETCH_SIZE/WRITE_SIZE."""
    import torch

    n = megabytes * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy probe: {megabytes} MiB read + {megabytes} MiB written")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_rate(A, h, c, threads, seconds_target):
    """Components/s of the oracle on `threads` host threads over a prefix of the workload sized for
    about seconds_target (calibrated on a short prefix)."""
    import oracle

    block = c["block"]
    k_cal = 8 if block in (0, 1) else c["block"]
    t0 = time.perf_counter()
    oracle.decompose(A, c["mu"], c["tau"], h, c["als_iters"], block, threads=threads, k_limit=k_cal)
    per = (time.perf_counter() - t0) / k_cal
    k_s = int(max(k_cal, min(4096, seconds_target / max(per, 1e-9))))
    if block not in (0, 1):
        k_s = max(block, (k_s // block) * block)
    t0 = time.perf_counter()
    r = oracle.decompose(A, c["mu"], c["tau"], h, c["als_iters"], block, threads=threads, k_limit=k_s)
    dt = time.perf_counter() - t0
    done = len(r["D"])
    return done / dt, done, dt


def cpu_baseline(A, h, c, seconds_target=15.0):
    """The oracle as it stands on the host cores, over a bounded prefix of the same workload (the
    same weights as the GPU run)."""
    threads = min(len(os.sched_getaffinity(0)), 16)
    v, done, dt = oracle_rate(A, h, c, threads, seconds_target)
    return {"value": v, "unit": "components/s", "cores": threads, "kind": "oracle",
            "sample": f"first {done} components of the same workload ({dt:.1f} s wall)",
            "cpu_model": cpu_model()}


def oracle_timings():
    """The plain oracle single-threaded and on all host cores (up to 16) on the small workloads and
    on a prefix of the 2560 x 2560 one; one JSON line."""
    from expanded_rank_matrix_amd import inputs

    cores = min(len(os.sched_getaffinity(0)), 16)
    rows = []
    for name, budget in (("tiny64x48", 5.0), ("lowrank1024", 20.0), ("attn2560", 20.0)):
        c = inputs.CONFIGS[name]
        A, h = inputs.make_input(name)
        for threads in (1, cores):
            v, done, dt = oracle_rate(A, h, c, threads, budget)
            rows.append({"workload": name, "threads": threads, "components_per_s": v, "components": done,
                         "seconds": dt})
            log(f"oracle {name} threads={threads}: {v:.1f} components/s over {done} components ({dt:.1f} s)")
    print(json.dumps({"oracle_timings": rows, "cpu_model": cpu_model(), "cores": cores}), flush=True)


def bandwidth_probe():
    """Sustained read and copy bandwidth of buffers inside and beyond the 256 MB Infinity Cache
    (26 MB is the 2560 x 2560 residual, 100 MB the 9728 x 2560 one): a sum reads the buffer once, a
    copy reads and writes it.  Repeated back to back, a buffer that fits stays in the cache."""
    import torch

    out = []
    for mb in (26, 100, 1024):
        n = mb * (1 << 20) // 4
        x = torch.randn(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        reps = max(20, int(4096 / mb))
        for _ in range(3):
            x.sum()
            y.copy_(x)
        torch.cuda.synchronize()
        res = {"MB": mb}
        for kind in ("read", "copy"):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                if kind == "read":
                    x.sum()
                else:
                    y.copy_(x)
            e1.record()
            torch.cuda.synchronize()
            sec = e0.elapsed_time(e1) * 1e-3 / reps
            nbytes = 4.0 * n * (1 if kind == "read" else 2)
            res[kind + "_GBps"] = nbytes / sec / 1e9
        log(f"probe {mb} MB: read {res['read_GBps']:.0f} GB/s, copy {res['copy_GBps']:.0f} GB/s")
        out.append(res)
        del x, y
    print(json.dumps({"bandwidth_probe": out, "note": "torch sum (read once) and copy_ (read + write), "
                      "buffers repeated back to back; 26 and 100 MB fit the 256 MB Infinity Cache"}), flush=True)


def factor_sparsity(out, m, n):
    """Zero fractions of B and C and the effective bits per weight of the mask+sign storage,
    (m k (2 - s_B) + k n (2 - s_C)) / (m n), D absorbed (pith.science free parameters, Eq. 5);
    counted on the host from the emitted packed factors."""
    def zeros(packed, length):
        # a 2-bit code is nonzero iff either of its bits is set; tail codes are zero by the format
        w = packed.cpu().numpy().view(np.uint32)
        nonzero = int(np.bitwise_count((w | (w >> np.uint32(1))) & np.uint32(0x55555555)).sum())
        return w.shape[0] * length - nonzero
    k = out["D"].shape[0]
    sB = zeros(out["B"], m) / (m * k)
    sC = zeros(out["C"], n) / (k * n)
    bpw = (m * k * (2.0 - sB) + k * n * (2.0 - sC)) / (m * n)
    return {"zero_fraction_B": sB, "zero_fraction_C": sC, "bpw": bpw, "bpw_with_D": bpw + 32.0 * k / (m * n)}


def infer_bench(args, erm, torch, A, h, c, k, m, n, out, stream):
    """Inference y = B diag(D) C x from the packed factors of one decomposition of the workload
    (decomposed once, untimed); each step is one externd_apply_factors call on `batch` vectors
    already in HBM.  The roofline counts the packed factors, D, x and y once per call."""
    erm.decompose(A, c["mu"], c["tau"], h, c["als_iters"], c["block"], stream=stream, out=out)
    X = torch.randn((args.batch, n), dtype=torch.float32, device="cuda")
    Y = torch.empty((args.batch, m), dtype=torch.float32, device="cuda")
    # --static: the allocation-free entry point (its kernels only, on the file-scope workspace)
    call = erm.apply_factors_static if args.static else erm.apply_factors
    for _ in range(max(1, args.warmup)):
        call(out["B"], out["C"], out["D"], m, n, X, stream=stream, out=Y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        call(out["B"], out["C"], out["D"], m, n, X, stream=stream, out=Y)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1) / args.steps
    nbytes = 4.0 * (out["B"].numel() + out["C"].numel() + k) + 4.0 * args.batch * (m + n)
    achieved = nbytes / (gpu_ms * 1e-3) / 1e9
    res = {
        "metric": f"packed-factor inference vectors/s ({m}x{n}, k={k})",
        "value": args.batch * args.steps / wall,
        "unit": "vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"infer_{args.workload}", "m": m, "n": n, "k": k, "batch": args.batch,
                   "factors": "packed 2-bit B and C of one decomposition of the workload",
                   "entry": "externd_apply_factors_static" if args.static else "externd_apply_factors"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "infer_c + infer_b + infer_reduce (one call)", "gpu_ms_per_call": gpu_ms,
                     "bytes_per_call": nbytes},
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="attn2560")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="run a plain copy of this many MiB first (counter calibration)")
    ap.add_argument("--infer", action="store_true",
                    help="time inference from the workload's packed factors instead of the decomposition")
    ap.add_argument("--batch", type=int, default=1, help="vectors per inference call (--infer)")
    ap.add_argument("--static", action="store_true",
                    help="--infer through the allocation-free entry point (no per-call workspace)")
    ap.add_argument("--sweeps", type=int, default=0, help="refinement sweeps after the greedy pass")
    ap.add_argument("--energy-target", type=float, default=0.0,
                    help="stop at the first component whose energy reaches this value")
    ap.add_argument("--safeguard", action="store_true", help="Prop. 2 single-entry safeguard")
    ap.add_argument("--block", type=int, default=None, help="override the workload's block size")
    ap.add_argument("--mu", type=float, default=None, help="override the workload's mu")
    ap.add_argument("--ablation", type=int, default=0,
                    help="1: block targets without decorrelation, 2: unweighted V-step projection")
    ap.add_argument("--residual-hbm", action="store_true",
                    help="sequential path: keep the residual in HBM even where it fits in LDS")
    ap.add_argument("--probe", action="store_true", help="bandwidth probe only")
    ap.add_argument("--oracle-timings", action="store_true", help="oracle timings only (host)")
    args = ap.parse_args()
    if args.oracle_timings:
        oracle_timings()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build runs the "
              "decomposition on a single MI355X", file=sys.stderr)
        sys.exit(2)

    import torch

    import expanded_rank_matrix_amd as erm
    from expanded_rank_matrix_amd import inputs

    if args.probe:
        bandwidth_probe()
        return
    if args.copy_mb > 0:
        copy_probe(args.copy_mb)
    c = dict(inputs.CONFIGS[args.workload])
    if args.block is not None:
        c["block"] = args.block
    if args.mu is not None:
        c["mu"] = args.mu
    options = dict(energy_target=args.energy_target, safeguard=args.safeguard, sweeps=args.sweeps,
                   ablation=args.ablation, residual_hbm=args.residual_hbm)
    # not the workload as defined
    variant = any(options.values()) or args.block is not None or args.mu is not None
    A_np, h_np = inputs.make_input(args.workload)
    m, n = A_np.shape
    A = torch.from_numpy(A_np).cuda()
    h = None if h_np is None else torch.from_numpy(h_np).cuda()
    k = erm.rank(m, n, c["mu"])
    out = dict(B=torch.empty((k, erm.packed_words(m)), dtype=torch.int32, device="cuda"),
               C=torch.empty((k, erm.packed_words(n)), dtype=torch.int32, device="cuda"),
               D=torch.empty(k, dtype=torch.float32, device="cuda"),
               energy=torch.empty(k, dtype=torch.float64, device="cuda"))
    stream = torch.cuda.current_stream()
    if args.infer:
        infer_bench(args, erm, torch, A, h, c, k, m, n, out, stream)
        return
    for _ in range(args.warmup):
        erm.decompose(A, c["mu"], c["tau"], h, c["als_iters"], c["block"], stream=stream, out=out, **options)
    torch.cuda.synchronize()
    kernel_ms, stats = [], None
    t0 = time.perf_counter()
    for _ in range(args.steps):
        r = erm.decompose(A, c["mu"], c["tau"], h, c["als_iters"], c["block"], stream=stream, out=out,
                          **options)
        stats = r["stats"]
        kernel_ms.append(stats["kernel_ms"])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    # components fitted: with an energy target only the kept ones, each sweep refits them again
    fits = stats["components_used"] * (1 + args.sweeps)
    value = fits * args.steps / wall
    kms = float(np.mean(kernel_ms))
    energy = out["energy"].cpu().numpy()
    # the traffic record was taken on the workload as defined; a variant has none
    traffic = None if variant else measured_traffic(args.workload)
    if c["block"] in (0, 1):
        achieved = stats["bytes_algorithmic"] / (kms * 1e-3) / 1e9
        lds = bool(stats["residual_lds"])
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                "kernel": "seq_kernel (persistent)", "kernel_ms": kms,
                "bytes_per_launch": stats["bytes_algorithmic"],
                "achieved_is": "algorithmic residual bytes / kernel time (the effective rate)",
                "residual_served_by": ("R rows from each workgroup's LDS, R^T from L2/HBM" if lds
                                       else "R and R^T from L2/HBM"),
                "limiter": "latency: 2T + 1 dependent grid-wide exchanges and exact selections per component"}
        if traffic is not None:
            roof["counter_GBps"] = traffic / (kms * 1e-3) / 1e9
    else:
        # The block path's contractions run on int8 MFMA with R in fixed point; they stream R once
        # each, so the bound is HBM.  The fp64-equivalent rate of the same work is reported beside.
        achieved = stats["bytes_algorithmic"] / (kms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                "kernel": "block-ALS path (all kernels)", "kernel_ms": kms,
                "bytes_per_launch": stats["bytes_algorithmic"],
                "fp64_equivalent_tflops": stats["flops_algorithmic"] / (kms * 1e-3) / 1e12}
    res = {
        "metric": "ExTernD components fitted/sec + achieved GB/s at 2560x2560, mu=3",
        "source_digest": source_digest("seq" if c["block"] in (0, 1) else "block"),
        "value": value,
        "unit": "components/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "m": m, "n": n, "mu": c["mu"], "k": k, "tau": c["tau"],
                   "als_iters": c["als_iters"], "block": c["block"],
                   "residual": (("fp32, rows resident in each workgroup's LDS, transpose in HBM; fp64 sums"
                                 if stats["residual_lds"] else "fp32 in HBM (both copies); fp64 sums")
                                if c["block"] in (0, 1) else
                                "fp32 in HBM; contractions exact on its 48-bit fixed-point image (int8 MFMA)"),
                   "energy_final": float(energy[-1]),
                   "passes": stats["passes"], "early_exits": stats["early_exits"]},
        "roofline": roof,
    }
    if variant:
        res["config"]["options"] = dict(options, block=c["block"], mu=c["mu"])
        res["config"]["components_used"] = stats["components_used"]
        res["config"]["fits_per_decomposition"] = fits
        res["config"]["safeguard_activations"] = stats["safeguard_activations"]
        res["config"]["sweep_reverts"] = stats["sweep_reverts"]
    if c["block"] not in (0, 1):
        res["config"].update(factor_sparsity(out, m, n))
    if c["block"] in (0, 1) and k >= 256:
        res["config"]["energy_every_256"] = [float(energy[i]) for i in range(255, k, 256)]
    if not args.no_cpu and not variant:
        res["cpu_baseline"] = cpu_baseline(A_np, h_np, c)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
