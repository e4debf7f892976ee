"""Benchmark of the batched Muon step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one muon_step_batched call over the whole batch: momentum, Frobenius
normalization, 5 Newton-Schulz iterations and the weight update for every
matrix, on synthetic seeded inputs already resident in HBM.  The default
workload is 96 bf16 expert matrices of 2048 x 6144.  Prints one JSON line.

The per-kernel durations come from HIP events that the library records around
each launch on the same stream during the timed region.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from newton_schulz_03_amd import rocprof_summary  # noqa: E402  (plain Python, loads no library)

METRIC = "expert matrices orthogonalized/sec + % bf16 MFMA peak (6144×2048, 5 NS steps)"
# HBM traffic of the product kernel per launch, from hardware counters (FETCH_SIZE and
# WRITE_SIZE, scaled by a copy of known size); used while the kernel sources are unchanged
TRAFFIC_WORKLOAD = "c2_96x2048x6144"
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_prod_c2_96x2048x6144.md")
PEAK_TFLOPS = {"bf16": 2516.6, "fp32": 157.3}  # dense matrix-core peaks at 2.4 GHz
PEAK_HBM_GBS = 8000.0


def ns_flops(shape, steps, with_square=True):
    """Algorithmic flops of `steps` iterations: symmetric products count unique entries only."""
    s, l = min(shape), max(shape)
    gram = s * (s + 1) * l
    square = s * s * (s + 1) if with_square else 0
    prod = 2 * s * s * l
    return steps * (gram + square + prod), steps * gram, steps * square, steps * prod


def elementwise_bytes(shape, esize, call, nesterov):
    """Algorithmic HBM bytes of the three bandwidth-bound kernels, per matrix."""
    n = shape[0] * shape[1] * esize
    if call == "step":
        # read G, M, write M';  read M' (and G), write X0;  read O, W, write W'
        return 3 * n, (3 if nesterov else 2) * n, 3 * n
    # read X;  read X, write X0;  read O, write out
    return n, 2 * n, 2 * n


def make_inputs(wl, device, threads=16):
    import concurrent.futures

    import torch

    import workloads

    def one(j):
        raw = workloads.matrix_inputs(wl, j)
        return j, {k: workloads.cast(v, wl.dtype) for k, v in raw.items()}

    out = [None] * wl.batch
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        for j, d in ex.map(one, range(wl.batch)):
            out[j] = {k: v.to(device) for k, v in d.items()}
    torch.cuda.synchronize(device)
    return out


def cpu_baseline(wl, seconds: float, max_sample: int):
    """The float64 oracle on the first matrices of the same workload, timed on the host.

    Matrices are run one after another until `seconds` of oracle time have
    passed (at least one, at most `max_sample`); input generation is not timed.
    """
    import numpy as np

    import oracle
    import workloads

    try:
        from threadpoolctl import threadpool_info

        cores = max(int(i.get("num_threads", 1)) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:  # pragma: no cover - threadpoolctl missing
        cores = os.cpu_count() or 1
    dt = 0.0
    sample = 0
    while sample < min(max_sample, wl.batch) and (sample == 0 or dt < seconds):
        raw = workloads.matrix_inputs(wl, sample)
        h = {k: workloads.as_float64(workloads.cast(v, wl.dtype)) for k, v in raw.items()}
        t0 = time.perf_counter()
        if wl.call == "step":
            oracle.muon_step(h["w"], h["g"], h["m"], lr=wl.lr, beta=wl.beta, nesterov=wl.nesterov,
                             steps=wl.steps, coeffs=wl.coeffs, eps=wl.eps)
        else:
            oracle.newton_schulz(h["x"], wl.steps, wl.coeffs, wl.eps)
        dt += time.perf_counter() - t0
        sample += 1
    shapes = sorted({tuple(s) for s in wl.shapes[:sample]})
    return {"value": round(sample / dt, 4), "unit": "matrices/s", "cores": cores, "kind": "oracle",
            "sample": f"first {sample} of {wl.batch} matrices {shapes} of {wl.name}, full step "
                      f"in float64 numpy, {dt:.1f} s of oracle time", "seconds": round(dt, 2)}


def adamw_bytes_per_element(dtype: str) -> int:
    """Algorithmic HBM bytes of one AdamW element: read p, g, m, v; write p, m, v."""
    e = 2 if dtype == "bf16" else 4
    return 3 * e + 4 * 4


def bench_adamw(args, wl) -> int:
    """One AdamW step per timed step over the workload's tensors (all resident in HBM)."""
    import concurrent.futures

    import torch

    import newton_schulz_03_amd as nsa
    import workloads

    dev = torch.device("cuda:0")

    def one(j):
        raw = workloads.adamw_inputs(wl, j)
        return j, {"p": workloads.cast(raw["p"], wl.dtype), "g": workloads.cast(raw["g"], wl.dtype),
                   "m": torch.from_numpy(raw["m"]), "v": torch.from_numpy(raw["v"])}

    print(f"[bench] generating {wl.name}: {wl.batch} tensors", file=sys.stderr, flush=True)
    ins = [None] * wl.batch
    with concurrent.futures.ThreadPoolExecutor(max_workers=16) as ex:
        for j, d in ex.map(one, range(wl.batch)):
            ins[j] = {k: v.to(dev) for k, v in d.items()}
    torch.cuda.synchronize(dev)
    P, G, M, V = ([d[k] for d in ins] for k in "pgmv")
    ws_bytes = nsa.adamw_workspace_bytes(wl.numels)
    raw_ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)
    off = (-raw_ws.data_ptr()) % 256
    ws = raw_ws[off:off + ws_bytes]

    def step():
        nsa.adamw_batched(P, G, M, V, lr=wl.lr, betas=(wl.beta1, wl.beta2), eps=wl.eps,
                          weight_decay=wl.weight_decay, step=wl.step, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    nsa.timing_reset()
    nsa.timing_enable(True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize(dev)
    nsa.timing_enable(False)
    kern = nsa.timing_read()
    total_ms = start.elapsed_time(end)
    n = sum(wl.numels)
    bpe = adamw_bytes_per_element(wl.dtype)
    k_ms = kern["adamw"][0] / max(1, kern["adamw"][1])
    gbs = n * bpe / (k_ms * 1e-3) / 1e9
    result = {
        "metric": "AdamW parameters updated/sec (non-expert parameters)",
        "value": round(n * args.steps / (total_ms * 1e-3), 1),
        "unit": "elements/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "tensors": wl.batch, "elements": n,
                   "moments": "fp32", "lr": wl.lr, "betas": [wl.beta1, wl.beta2],
                   "weight_decay": wl.weight_decay, "step": wl.step},
        "roofline": {"bound": "hbm", "kernel": "adamw", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": None, "bytes_per_element": bpe},
    }
    if not args.no_cpu_baseline:
        import numpy as np

        import oracle

        print(f"[bench] timing the oracle for about {args.cpu_seconds:.0f} s", file=sys.stderr,
              flush=True)
        done, dt, j = 0, 0.0, 0
        while dt < args.cpu_seconds and j < wl.batch:
            raw = workloads.adamw_inputs(wl, j)
            h = {k: workloads.as_float64(workloads.cast(v, wl.dtype)) if k in "pg" else
                 raw[k].astype(np.float64) for k, v in raw.items()}
            t0 = time.perf_counter()
            oracle.adamw_step(h["p"], h["g"], h["m"], h["v"], lr=wl.lr, beta1=wl.beta1,
                              beta2=wl.beta2, eps=wl.eps, weight_decay=wl.weight_decay,
                              step=wl.step)
            dt += time.perf_counter() - t0
            done += wl.numels[j]
            j += 1
        result["cpu_baseline"] = {"value": round(done / dt, 1), "unit": "elements/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": f"first {j} of {wl.batch} tensors ({done} elements), "
                                            f"float64 numpy, {dt:.1f} s"}
    print(json.dumps(result), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="c2_96x2048x6144")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle time for the CPU baseline (whole matrices, at least one)")
    ap.add_argument("--cpu-max-sample", type=int, default=64, help="most matrices timed on the oracle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--momentum-host", action="store_true",
                    help="keep the momentum in pinned host memory (the GPU reads and writes it "
                         "in place over the host link)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a known "
                         "byte count for scaling hardware traffic counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library orthogonalizes a ragged batch on a single "
              "MI355X and has no multi-GPU path (matrices are independent, so each rank would run "
              "its own share of whole matrices).", file=sys.stderr)
        return 2

    import torch

    import newton_schulz_03_amd as nsa
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    nsa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    adamw = workloads.adamw_workloads()
    if args.workload in adamw:
        return bench_adamw(args, adamw[args.workload])
    wl = workloads.standard_workloads()[args.workload]
    print(f"[bench] generating {wl.name}: {wl.batch} matrices", file=sys.stderr, flush=True)
    t0 = time.time()
    ins = make_inputs(wl, dev)
    print(f"[bench] inputs resident in HBM after {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    shapes = list(wl.shapes)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    ws = nsa.allocate_workspace(shapes, tdt, dev)
    c = wl.coeffs[2]

    if wl.call == "step":
        W = [d["w"] for d in ins]
        G = [d["g"] for d in ins]
        M = [d["m"] for d in ins]
        if args.momentum_host:
            M = [m.cpu().pin_memory() for m in M]
            for d in ins:
                del d["m"]
            torch.cuda.synchronize(dev)
            print("[bench] momentum moved to pinned host memory", file=sys.stderr, flush=True)

        def step():
            nsa.step_batched(W, G, M, lr=wl.lr, beta=wl.beta, nesterov=wl.nesterov,
                             steps=wl.steps, coeffs=wl.coeffs, eps=wl.eps, workspace=ws,
                             momentum_host=args.momentum_host)
    else:
        X = [d["x"] for d in ins]
        OUT = [torch.empty_like(x) for x in X]

        def step():
            nsa.ns_batched(X, steps=wl.steps, coeffs=wl.coeffs, eps=wl.eps, out=OUT, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    nsa.timing_reset()
    nsa.timing_enable(True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize(dev)
    nsa.timing_enable(False)
    kern = nsa.timing_read()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    esize = 2 if wl.dtype == "bf16" else 4
    fl = [ns_flops(s, wl.steps, c != 0.0) for s in shapes]
    alg_total = sum(f[0] for f in fl)
    alg_prod_launch = sum(2 * min(s) ** 2 * max(s) for s in shapes)
    alg_gram_launch = sum(min(s) * (min(s) + 1) * max(s) for s in shapes)
    alg_poly_launch = sum(min(s) ** 2 * (min(s) + 1) for s in shapes)
    peak = PEAK_TFLOPS[wl.dtype]

    def avg(name):
        ms, n = kern[name]
        return ms / n if n else float("nan")

    prod_ms = avg("prod")
    achieved = alg_prod_launch / (prod_ms * 1e-3) / 1e12
    per_kernel = {k: {"avg_ms": round(avg(k), 4), "launches": kern[k][1]} for k in nsa.KERNELS
                  if kern[k][1]}
    ns_ms = (kern["gram"][0] + kern["poly"][0] + kern["prod"][0]) / args.steps
    ew = [elementwise_bytes(s, esize, wl.call, wl.nesterov) for s in shapes]
    for name, idx in (("reduce", 0), ("normalize", 1), ("finish", 2)):
        if name not in per_kernel:
            continue
        b = sum(e[idx] for e in ew)
        per_kernel[name]["gbs"] = round(b / (avg(name) * 1e-3) / 1e9, 1)
        per_kernel[name]["hbm_frac"] = round(b / (avg(name) * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)
    for name, flops in (("gram", alg_gram_launch), ("poly", alg_poly_launch), ("prod", alg_prod_launch)):
        if kern[name][1]:
            t = flops / (avg(name) * 1e-3) / 1e12
            per_kernel[name]["tflops"] = round(t, 1)
            per_kernel[name]["mfma_frac"] = round(t / peak, 3)

    value = wl.batch * args.steps / (total_ms * 1e-3)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "shapes": sorted({tuple(s) for s in shapes}),
                   "ns_steps": wl.steps, "coeffs": list(wl.coeffs), "call": wl.call,
                   "nesterov": wl.nesterov, "lr": wl.lr, "beta": wl.beta,
                   "momentum": "pinned host memory" if args.momentum_host else "HBM"},
        "roofline": {"bound": "mfma", "kernel": "prod (X <- aX + BX)", "achieved": round(achieved, 1),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": rocprof_summary.read_traffic(TRAFFIC_SUMMARY, wl.name)
                     if wl.name == TRAFFIC_WORKLOAD else None},
        "ns_effective_tflops": round(alg_total / (total_ms / args.steps * 1e-3) / 1e12, 1),
        "ns_mfma_frac_whole_step": round(alg_total / (total_ms / args.steps * 1e-3) / 1e12 / peak, 4),
        "ns_kernels_ms_per_step": round(ns_ms, 3),
        "kernels": per_kernel,
    }
    if args.copy_calibration_mb > 0:
        # one plain copy of known size (reads n bytes, writes n bytes): hardware
        # traffic counters of the same run are scaled by what they read for it
        n = args.copy_calibration_mb * (1 << 20)
        src = torch.full((n // 4,), 1.5, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize(dev)
        result["copy_calibration_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline:
        print(f"[bench] timing the oracle for about {args.cpu_seconds:.0f} s", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, args.cpu_max_sample)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
