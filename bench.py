"""Benchmark of the batched Muon step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one muon_step_batched call over the whole batch: momentum, Frobenius
normalization, 5 Newton-Schulz iterations and the weight update for every
matrix, on synthetic seeded inputs already resident in HBM.  The default
workload is 96 bf16 expert matrices of 2048 x 6144.  Prints one JSON line.

The headline is timed with HIP events around the K steps alone, with the
library's per-kernel instrumentation off.  The per-kernel durations come from a
second pass of K steps in which the library records HIP events around each
launch, on the stream the kernels run on.  After them, on the same inputs,
"variants" times the step with e4m3 operands in the first two Newton-Schulz
steps and with the momentum in pinned host memory (not the headline; skipped
with --no-variants).

    python bench.py --hbm-ceiling

measures the plain HBM stream (1 and 2 reads, 1 and 2 writes, 16-byte
lane-contiguous vectors, with and without the nontemporal hint) that the
bandwidth-bound kernels are held against.

    python bench.py --tile-timeline [--workload NAME]

reads the per-workgroup timeline of the matrix-core launches from the
library's timeline build: how busy the CUs were, the idle time between tiles
and at the end of each launch, and each XCD's share.
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
PEAK_TFLOPS = {"bf16": 2516.6, "fp32": 157.3, "e4m3": 5033.2}  # dense matrix-core peaks, 2.4 GHz
PEAK_HBM_GBS = 8000.0


def ns_flops(shape, steps, with_square=True):
    """Algorithmic flops of `steps` iterations: symmetric products count unique entries only."""
    s, l = min(shape), max(shape)
    gram = s * (s + 1) * l
    square = s * s * (s + 1) if with_square else 0
    prod = 2 * s * s * l
    return steps * (gram + square + prod), steps * gram, steps * square, steps * prod


def elementwise_bytes(shape, esize, call):
    """Algorithmic HBM bytes of the two bandwidth-bound kernels, per matrix:
    prepare (which writes U into the iterate, zero padded to 256 on both
    sides) and finish."""
    n = shape[0] * shape[1] * esize
    pad = -(-shape[0] // 256) * 256 * (-(-shape[1] // 256) * 256) * esize
    if call == "step":
        # read G, M, write M' and the iterate;  read O, W, write W'
        return 3 * n + pad, 3 * n
    # read X, write the iterate;  read O, write out
    return n + pad, 2 * n


def make_inputs(wl, device, threads=16):
    import concurrent.futures

    import torch

    import workloads

    if wl.kind == "illcond":
        # the QR behind these inputs is slow on the host at 6144: build them on the device
        out = [workloads.illcond_inputs_device(wl, j, device)[0] for j in range(wl.batch)]
        torch.cuda.synchronize(device)
        return out

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
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - not Linux
        affinity = os.cpu_count() or 1
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
    return {"value": round(sample / dt, 4), "unit": "matrices/s", "cores": cores,
            "host_cpus": os.cpu_count(), "cpus_in_affinity": affinity, "kind": "oracle",
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


def bench_hbm_ceiling(args) -> int:
    """The plain HBM stream of the library's measurement kernel, per pattern:
    GB/s and the fraction of 8 TB/s, median of `steps` launches over buffers
    of the momentum pass's per-tensor size on the benchmark workload."""
    import torch

    import newton_schulz_03_amd as nsa

    dev = torch.device("cuda:0")
    n = args.hbm_bytes
    bufs = [torch.empty(n, dtype=torch.uint8, device=dev).fill_(k + 1) for k in range(4)]
    out = {}
    for n_in, n_out in ((1, 1), (2, 1), (2, 2)):
        for nt in (False, True):
            ins, outs = bufs[:n_in], bufs[2:2 + n_out]
            for _ in range(max(1, args.warmup)):
                nsa.hbm_stream(ins, outs, nontemporal=nt)
            times = []
            for _ in range(args.steps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                nsa.hbm_stream(ins, outs, nontemporal=nt)
                b.record()
                torch.cuda.synchronize(dev)
                times.append(a.elapsed_time(b))
            ms = sorted(times)[len(times) // 2]
            gbs = (n_in + n_out) * n / (ms * 1e-3) / 1e9
            out[f"{n_in}r{n_out}w{'_nt' if nt else ''}"] = {
                "ms": round(ms, 4), "gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}
    for k in range(2):
        assert torch.equal(bufs[2 + k], bufs[k])  # the last (2r2w) copy moved every byte
    print(json.dumps({"metric": "HBM read+write stream ceiling (plain copy kernel)",
                      "unit": "GB/s", "bytes_per_stream": n, "peak": PEAK_HBM_GBS,
                      "median_of": args.steps, "patterns": out}), flush=True)
    return 0


def bench_variants(args, wl, W, G, M, shapes, dev) -> dict:
    """The same step with its two options, after the headline and on the same
    inputs: e4m3 operands in the first two Newton-Schulz steps, and the
    momentum in pinned host memory.  Each: `warmup` untimed steps, then `steps`
    timed ones; not the headline (another dtype, or another memory)."""
    import torch

    import newton_schulz_03_amd as nsa

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize(dev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            fn()
        b.record()
        torch.cuda.synchronize(dev)
        return a.elapsed_time(b) / args.steps

    kw = dict(lr=wl.lr, beta=wl.beta, nesterov=wl.nesterov, steps=wl.steps, coeffs=wl.coeffs,
              eps=wl.eps)
    out = {}
    ws8 = nsa.allocate_workspace(shapes, torch.bfloat16, dev, fp8=True)
    ms = timed(lambda: nsa.step_batched(W, G, M, workspace=ws8, fp8_steps=2, **kw))
    out["fp8_steps_2"] = {"ms_per_step": round(ms, 3), "value": round(wl.batch / ms * 1e3, 2),
                          "unit": "matrices/s", "dtype": "bf16+e4m3"}
    print(f"[bench] variant e4m3 steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)
    del ws8
    mh = [m.cpu().pin_memory() for m in M]
    wsh = nsa.allocate_workspace(shapes, torch.bfloat16, dev, momentum_host=True)
    ms = timed(lambda: nsa.step_batched(W, G, mh, workspace=wsh, momentum_host=True, **kw))
    out["momentum_host"] = {"ms_per_step": round(ms, 3), "value": round(wl.batch / ms * 1e3, 2),
                            "unit": "matrices/s", "momentum": "pinned host memory"}
    print(f"[bench] variant momentum in host memory: {ms:.3f} ms/step", file=sys.stderr, flush=True)
    del wsh, mh
    torch.cuda.empty_cache()
    return out


def bench_link_ceiling(args) -> int:
    """The host link with plain DMA copies between pinned host memory and HBM, in
    the momentum's tensor sizes on the benchmark workload (96 bf16 tensors of
    2048 x 6144): host to device, device to host, and both at once on two
    streams; then the same two copies concurrent with an orthogonalization of
    the 96 matrices.  The lower bound of a step with the momentum in host
    memory is the time to move it both ways."""
    import torch

    import newton_schulz_03_amd as nsa

    dev = torch.device("cuda:0")
    n, per = 96, 2048 * 6144
    host = [torch.empty(per, dtype=torch.bfloat16).pin_memory() for _ in range(n)]
    back = [torch.empty(per, dtype=torch.bfloat16).pin_memory() for _ in range(n)]
    devb = [torch.empty(per, dtype=torch.bfloat16, device=dev) for _ in range(n)]
    devc = [torch.empty(per, dtype=torch.bfloat16, device=dev) for _ in range(n)]
    s_in, s_out = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    gb = n * per * 2 / 1e9

    def h2d():
        with torch.cuda.stream(s_in):
            for h, d in zip(host, devb):
                d.copy_(h, non_blocking=True)

    def d2h():
        with torch.cuda.stream(s_out):
            for h, d in zip(back, devc):
                h.copy_(d, non_blocking=True)

    xs = [torch.randn(2048, 6144, device=dev).to(torch.bfloat16) for _ in range(n)]
    outs = [torch.empty_like(x) for x in xs]
    ws = nsa.allocate_workspace([(2048, 6144)] * n, torch.bfloat16, dev)

    def ns():
        nsa.ns_batched(xs, steps=5, out=outs, workspace=ws)

    def best_ms(fn):
        times = []
        for _ in range(max(2, args.steps)):
            torch.cuda.synchronize(dev)
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize(dev)
            times.append((time.perf_counter() - t0) * 1e3)
        return sorted(times)[len(times) // 2]

    res = {}
    for name, fn, vol in (("h2d", h2d, gb), ("d2h", d2h, gb), ("both", lambda: (h2d(), d2h()), 2 * gb)):
        fn()
        ms = best_ms(fn)
        res[name] = {"ms": round(ms, 2), "gbs": round(vol / ms * 1e3, 1)}
        print(f"[bench] link {name}: {ms:.1f} ms", file=sys.stderr, flush=True)
    ns()
    res["ns_alone"] = {"ms": round(best_ms(ns), 2)}
    res["ns_with_both_copies"] = {"ms": round(best_ms(lambda: (h2d(), d2h(), ns())), 2)}
    print(json.dumps({"metric": "host link ceiling (pinned host memory <-> HBM, DMA copies)",
                      "unit": "GB/s", "bytes_each_way": n * per * 2, "tensors": n,
                      "median_of": max(2, args.steps), "patterns": res}), flush=True)
    return 0


def bench_blas_compare(args) -> int:
    """The vendor library's batched bf16 GEMM (torch.bmm, hipBLASLt) on the
    products of one Newton-Schulz step of the benchmark workload, beside this
    library's kernels on the same shapes: B X (2048x2048 @ 2048x6144), the full
    X X^T (2048x6144 @ 6144x2048, which the library forms as upper tiles only)
    and A A (2048^3), 96 of each, plus one 8192^3 product.  Medians of `steps`
    timed batches of 10 launches."""
    import torch

    import newton_schulz_03_amd as nsa

    dev = torch.device("cuda:0")
    n, s, l = 96, 2048, 6144
    peak = PEAK_TFLOPS["bf16"]
    Bm = torch.randn(n, s, s, device=dev).to(torch.bfloat16)
    X = torch.randn(n, s, l, device=dev).to(torch.bfloat16)
    XT = X.transpose(1, 2).contiguous()
    O = torch.empty(n, s, l, device=dev, dtype=torch.bfloat16)
    A = torch.empty(n, s, s, device=dev, dtype=torch.bfloat16)
    big = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    big_out = torch.empty_like(big)

    def med_ms(fn):
        fn()
        torch.cuda.synchronize(dev)
        times = []
        for _ in range(max(3, args.steps)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(10):
                fn()
            b.record()
            torch.cuda.synchronize(dev)
            times.append(a.elapsed_time(b) / 10)
        return sorted(times)[len(times) // 2]

    res = {}
    for name, fn, flops in (
            ("prod B@X", lambda: torch.bmm(Bm, X, out=O), n * 2 * s * s * l),
            ("gram X@X^T (full square)", lambda: torch.bmm(X, XT, out=A), n * 2 * s * s * l),
            ("A@A (full square)", lambda: torch.bmm(Bm, Bm, out=A), n * 2 * s ** 3),
            ("8192^3", lambda: torch.mm(big, big, out=big_out), 2 * 8192 ** 3)):
        ms = med_ms(fn)
        res[name] = {"ms": round(ms, 3), "tflops": round(flops / ms / 1e9, 1),
                     "frac": round(flops / ms / 1e9 / peak, 4)}
        print(f"[bench] torch {name}: {ms:.3f} ms", file=sys.stderr, flush=True)
    del Bm, XT, O, A, big, big_out
    xs = list(X.unbind(0))
    outs = [torch.empty_like(x) for x in xs]
    ws = nsa.allocate_workspace([(s, l)] * n, torch.bfloat16, dev)
    nsa.ns_batched(xs, steps=5, out=outs, workspace=ws)
    torch.cuda.synchronize(dev)
    nsa.timing_reset()
    nsa.timing_enable(True)
    for _ in range(max(3, args.steps)):
        nsa.ns_batched(xs, steps=5, out=outs, workspace=ws)
    torch.cuda.synchronize(dev)
    nsa.timing_enable(False)
    kern = nsa.timing_read()
    lib = {}
    for name, key, flops in (("prod B@X", "prod", n * 2 * s * s * l),
                             ("gram X@X^T (upper tiles)", "gram", n * s * (s + 1) * l),
                             ("A@A (upper tiles)", "poly", n * s * s * (s + 1))):
        ms = kern[key][0] / kern[key][1]
        lib[name] = {"ms": round(ms, 3), "tflops": round(flops / ms / 1e9, 1),
                     "frac": round(flops / ms / 1e9 / peak, 4)}
    print(json.dumps({"metric": "bf16 GEMM: vendor library (torch.bmm) against this library's kernels",
                      "unit": "TFLOP/s", "peak": peak, "batch": n, "note": "frac: algorithmic flops / "
                      "bf16 dense peak; the library's symmetric products count s(s+1) per row pair",
                      "torch": res, "library": lib}), flush=True)
    return 0


def _cu_masked_stream(mask_words):
    """A HIP stream restricted to the CUs set in `mask_words` (32-bit words), at the
    default priority; returned as (torch ExternalStream, raw handle)."""
    import ctypes

    import torch

    hip = ctypes.CDLL("libamdhip64.so")
    handle = ctypes.c_void_p()
    arr = (ctypes.c_uint32 * len(mask_words))(*mask_words)
    st = hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), ctypes.c_uint32(len(mask_words)), arr)
    if st != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask failed with status {st}")
    return torch.cuda.ExternalStream(handle.value), handle


def bench_overlap(args) -> int:
    """Dense-matrix orthogonalization on a second stream while expert GEMMs run.

    Expert load: bf16 products of the expert FFN shapes (tokens x 6144 by 6144 x
    2048, then tokens x 2048 by 2048 x 6144), repeated; dense load: one
    orthogonalization of the dense attention matrices (16 x 6144^2 + 16 x
    6144x1024, 5 steps).  Both at the default stream priority.  Times: each
    alone, both on two streams, and both on two streams with the CUs split
    between them (one CU in four for the dense work, by mask).
    """
    import torch

    import newton_schulz_03_amd as nsa
    import workloads

    dev = torch.device("cuda:0")
    wl = workloads.standard_workloads()["c4_dense_attn"]
    print(f"[bench] overlap: generating {wl.batch} dense matrices", file=sys.stderr, flush=True)
    X = [d["x"] for d in make_inputs(wl, dev)]
    OUT = [torch.empty_like(x) for x in X]
    ws = nsa.allocate_workspace(list(wl.shapes), torch.bfloat16, dev)
    tokens = 8192
    g = torch.Generator(device="cpu").manual_seed(7)
    act = torch.randn(tokens, 6144, generator=g).to(dev, torch.bfloat16)
    w_up = (torch.randn(6144, 2048, generator=g) * 0.02).to(dev, torch.bfloat16)
    w_down = (torch.randn(2048, 6144, generator=g) * 0.02).to(dev, torch.bfloat16)
    hid = torch.empty(tokens, 2048, device=dev, dtype=torch.bfloat16)
    out = torch.empty(tokens, 6144, device=dev, dtype=torch.bfloat16)
    reps = args.overlap_gemms

    def experts(stream):
        with torch.cuda.stream(stream):
            for _ in range(reps):
                torch.matmul(act, w_up, out=hid)
                torch.matmul(hid, w_down, out=out)

    def dense(stream, budget=0):
        with torch.cuda.stream(stream):
            nsa.ns_batched(X, steps=wl.steps, coeffs=wl.coeffs, eps=wl.eps, out=OUT, workspace=ws,
                           cu_budget=budget)

    def timed(fn):
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize(dev)
        return (time.perf_counter() - t0) * 1e3

    # a bandwidth-bound load standing in for the exchange traffic of the step
    # (weight gathers, gradient reduce-scatter): repeated 1 GiB device copies
    cp_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    cp_dst = torch.empty_like(cp_src)

    def copies(stream):
        with torch.cuda.stream(stream):
            for _ in range(args.overlap_copies):
                cp_dst.copy_(cp_src)

    sa, sb = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    for _ in range(args.warmup):
        timed(lambda: (experts(sa), dense(sb)))
        timed(lambda: (copies(sa), dense(sb)))
    t_exp = min(timed(lambda: experts(sa)) for _ in range(3))
    t_dense = min(timed(lambda: dense(sb)) for _ in range(3))
    t_both = min(timed(lambda: (experts(sa), dense(sb))) for _ in range(3))
    t_copy = min(timed(lambda: copies(sa)) for _ in range(3))
    t_copy_dense = min(timed(lambda: (copies(sa), dense(sb))) for _ in range(3))
    budget = args.overlap_cu_budget
    timed(lambda: (experts(sa), dense(sb, budget)))
    t_dense_b = min(timed(lambda: dense(sb, budget)) for _ in range(3))
    t_both_b = min(timed(lambda: (experts(sa), dense(sb, budget))) for _ in range(3))
    t_copy_b = min(timed(lambda: (copies(sa), dense(sb, budget))) for _ in range(3))
    ref = [o.clone() for o in OUT]
    dense(sb)
    torch.cuda.synchronize(dev)
    same = all(torch.equal(a, b) for a, b in zip(ref, OUT))
    result = {
        "metric": "dense-matrix orthogonalization overlapped with expert GEMMs (one GPU)",
        "value": round(t_exp + t_dense - t_both, 3),
        "unit": "ms saved by overlap",
        "n_gpus": 1, "steps": 3, "warmup": args.warmup, "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "c4_dense_attn + expert FFN products",
                   "expert_products": f"{reps} x ({tokens}x6144 @ 6144x2048, then @ 2048x6144)",
                   "streams": "two, default priority"},
        "ms": {"experts_alone": round(t_exp, 3), "dense_alone": round(t_dense, 3),
               "sum": round(t_exp + t_dense, 3), "both_two_streams": round(t_both, 3),
               "copies_alone": round(t_copy, 3),
               "copies_and_dense_two_streams": round(t_copy_dense, 3),
               "saved_against_copies": round(t_copy + t_dense - t_copy_dense, 3),
               f"dense_alone_cu_budget_{budget}": round(t_dense_b, 3),
               f"experts_and_dense_cu_budget_{budget}": round(t_both_b, 3),
               f"copies_and_dense_cu_budget_{budget}": round(t_copy_b, 3)},
        "copy_load": f"{args.overlap_copies} x 1 GiB device-to-device copies",
        "dense_output_identical_under_overlap": same,
    }
    try:
        n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
        words = (n_cu + 31) // 32
        dense_mask = [0] * words
        exp_mask = [0] * words
        for cu in range(n_cu):
            (dense_mask if cu % 4 == 3 else exp_mask)[cu // 32] |= 1 << (cu % 32)
        ma, ha = _cu_masked_stream(exp_mask)
        mb, hb = _cu_masked_stream(dense_mask)
        timed(lambda: (experts(ma), dense(mb)))
        t_mask = min(timed(lambda: (experts(ma), dense(mb))) for _ in range(3))
        dense(mb)
        torch.cuda.synchronize(dev)
        result["ms"]["both_cu_split_3_to_1"] = round(t_mask, 3)
        result["dense_output_identical_cu_split"] = all(torch.equal(a, b) for a, b in zip(ref, OUT))
    except Exception as e:  # a missing runtime entry point only removes this line
        result["cu_mask_error"] = str(e)
    print(json.dumps(result), flush=True)
    return 0 if same else 1


TRACE_LIB = os.path.join(ROOT, "newton_schulz_03_amd", "lib", "libmuon_mi355x_tiletrace.so")
TRACE_SLOTS = ("gram", "a2", "product_wide", "product_square")


def bench_tile_timeline(args, wl) -> int:
    """Per-workgroup timeline of the matrix-core launches of one orthogonalization
    of the workload's matrices (bf16), from the timeline build of the library
    (libmuon_mi355x_tiletrace.so: the same kernels plus a start and end stamp on
    the 100 MHz real-time counter and the hardware ids of the CU, per
    workgroup).  For the last launch of each kind (Gram, A^2, wide and square
    product) it reports how busy the CUs were over the launch, the idle time
    between consecutive tiles on one CU, the idle time at the end, the tiles
    and end time of each XCD, and how an off-diagonal tile's time splits into
    claim and prologue (until the first slice is in LDS), K loop (its first 8
    slices, the middle, the last 8) and epilogue (from the last slice to the
    stores issued)."""
    import ctypes

    import numpy as np
    import torch

    import newton_schulz_03_amd as nsa

    if wl.dtype != "bf16":
        print("--tile-timeline covers the bf16 kernels", file=sys.stderr)
        return 1
    lib = nsa.load_library(TRACE_LIB)
    if not hasattr(lib, "muon_tile_trace_read"):
        raise RuntimeError(f"{TRACE_LIB} is not the timeline build")
    dev = torch.device("cuda:0")
    gen = torch.Generator(device="cpu").manual_seed(wl.seed)
    xs = [torch.randn(*sh, generator=gen).to(torch.bfloat16).to(dev) for sh in wl.shapes]
    outs = [torch.empty_like(x) for x in xs]
    ws = nsa.allocate_workspace(list(wl.shapes), torch.bfloat16, dev)
    for _ in range(max(1, args.warmup)):
        nsa.ns_batched(xs, steps=wl.steps, coeffs=wl.coeffs, out=outs, workspace=ws)
    torch.cuda.synchronize(dev)
    if lib.muon_tile_trace_clear() != 0:
        raise RuntimeError("muon_tile_trace_clear failed")
    nsa.ns_batched(xs, steps=wl.steps, coeffs=wl.coeffs, out=outs, workspace=ws)
    torch.cuda.synchronize(dev)
    nslot, nblk, nword = len(TRACE_SLOTS), 65536, 7
    buf = np.zeros(nslot * nblk * nword, dtype=np.uint64)
    lib.muon_tile_trace_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    if lib.muon_tile_trace_read(buf.ctypes.data, buf.nbytes) != 0:
        raise RuntimeError("muon_tile_trace_read failed")
    buf = buf.reshape(nslot, nblk, nword)
    if args.timeline_raw:
        np.save(args.timeline_raw, buf)
    result = {"metric": "matrix-core launch timeline (one orthogonalization, last launch of each kind)",
              "workload": wl.name, "unit": "us", "launches": {}}
    for slot, name in enumerate(TRACE_SLOTS):
        rec = buf[slot]
        rec = rec[rec[:, 0] > 0]
        if len(rec) == 0:
            continue
        start, end = rec[:, 0].astype(np.int64), rec[:, 1].astype(np.int64)
        ids = rec[:, 2]
        tile = (ids & 0xFFFFFF).astype(np.int64) - 1
        xcd = ((ids >> 24) & 0xF).astype(np.int64)
        hw = (ids >> 32).astype(np.int64)
        cu = xcd * 256 + ((hw >> 8) & 0xFF)  # XCD, shader engine, CU
        work = tile >= 0
        t0, t1 = start.min(), end.max()
        span = (t1 - t0) / 100.0
        busy, gaps, tails, boundaries = [], 0.0, [], 0
        for k in np.unique(cu[work]):
            m = work & (cu == k)
            order = np.argsort(start[m])
            s_, e_ = start[m][order], end[m][order]
            busy.append(np.sum(e_ - s_) / 100.0)
            gaps += np.sum(s_[1:] - e_[:-1]) / 100.0
            boundaries += len(s_) - 1
            tails.append((t1 - e_[-1]) / 100.0)
        dur = (end[work] - start[work]) / 100.0
        # off-diagonal tiles: start -> K loop -> epilogue (claim and prologue, K loop, epilogue)
        kb, ke = rec[:, 3].astype(np.int64), rec[:, 4].astype(np.int64)
        k8, kl = rec[:, 5].astype(np.int64), rec[:, 6].astype(np.int64)
        ph = work & (kb > 0) & (ke >= kb)
        phases = None
        if np.any(ph):
            phases = {k: [round(float(np.percentile(v, q)), 2) for q in (10, 50, 90)] for k, v in (
                ("prologue", (kb[ph] - start[ph]) / 100.0), ("k_loop", (ke[ph] - kb[ph]) / 100.0),
                ("epilogue", (end[ph] - ke[ph]) / 100.0))}
            # tiles with at least 16 slices: first 8, middle, last 8 slices of the K loop
            sp = ph & (k8 >= kb) & (kl >= k8) & (ke >= kl)
            if np.any(sp):
                for k, v in (("k_first8", (k8[sp] - kb[sp]) / 100.0),
                             ("k_middle", (kl[sp] - k8[sp]) / 100.0),
                             ("k_last8", (ke[sp] - kl[sp]) / 100.0)):
                    phases[k] = [round(float(np.percentile(v, q)), 2) for q in (10, 50, 90)]
        result["launches"][name] = {
            "workgroups": int(len(rec)), "tiles": int(work.sum()), "cus": int(len(busy)),
            "truncated": bool(len(rec) >= nblk),  # a larger grid than the timeline holds
            "span": round(span, 1),
            "busy_fraction": round(float(np.mean(busy)) / span, 4),
            "tile_p10_median_p90": [round(float(np.percentile(dur, q)), 1) for q in (10, 50, 90)],
            "idle_between_tiles_per_cu": round(gaps / len(busy), 1),
            "idle_per_tile_boundary": round(gaps / max(boundaries, 1), 2),
            "idle_at_end_mean_max": [round(float(np.mean(tails)), 1), round(float(np.max(tails)), 1)],
            "phases_p10_median_p90": phases,
            "xcd_tiles": [int(np.sum(work & (xcd == x))) for x in range(8)],
            "xcd_last_end": [round(float((end[work & (xcd == x)].max() - t0) / 100.0), 1)
                             if np.any(work & (xcd == x)) else None for x in range(8)],
        }
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
    ap.add_argument("--overlap", action="store_true",
                    help="measure the dense-matrix orthogonalization overlapped with expert GEMMs")
    ap.add_argument("--overlap-gemms", type=int, default=120,
                    help="expert FFN product pairs in the overlap load")
    ap.add_argument("--overlap-cu-budget", type=int, default=64,
                    help="CUs the dense orthogonalization keeps in the budgeted overlap runs")
    ap.add_argument("--overlap-copies", type=int, default=100,
                    help="1 GiB device copies in the bandwidth-bound overlap load")
    ap.add_argument("--fp8-steps", type=int, default=0,
                    help="e4m3 operands in the first N Newton-Schulz steps (bf16 workloads; "
                         "the line is then labelled as such, not the bf16 headline)")
    ap.add_argument("--momentum-host", action="store_true",
                    help="keep the momentum in pinned host memory (the GPU reads and writes it "
                         "in place over the host link)")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="measure the plain HBM stream ceiling of the bandwidth-bound kernels")
    ap.add_argument("--hbm-bytes", type=int, default=96 * 2048 * 6144 * 2,
                    help="bytes per stream for --hbm-ceiling (default: one bf16 tensor of the "
                         "benchmark workload, 96 x 2048 x 6144)")
    ap.add_argument("--blas-compare", action="store_true",
                    help="time the vendor library's batched GEMM on the step's products beside "
                         "this library's kernels")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the step's e4m3 and host-momentum variants after the headline")
    ap.add_argument("--link-ceiling", action="store_true",
                    help="measure the host link with plain DMA copies of the momentum's size")
    ap.add_argument("--tile-timeline", action="store_true",
                    help="per-workgroup timeline of the matrix-core launches, from the library's "
                         "timeline build")
    ap.add_argument("--timeline-raw", default="",
                    help="with --tile-timeline: also save the raw per-workgroup records (numpy, "
                         "slots x workgroups x [start, end, ids, K loop start and end, slices 8 and nk-8])")
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
    if args.tile_timeline:  # loads the timeline build instead of the library
        torch.cuda.set_device(0)
        return bench_tile_timeline(args, workloads.standard_workloads()[args.workload])
    nsa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.overlap:
        return bench_overlap(args)
    if args.hbm_ceiling:
        return bench_hbm_ceiling(args)
    if args.link_ceiling:
        return bench_link_ceiling(args)
    if args.blas_compare:
        return bench_blas_compare(args)
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
    ws = nsa.allocate_workspace(shapes, tdt, dev, fp8=args.fp8_steps > 0,
                                momentum_host=args.momentum_host and wl.call == "step")
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
                             momentum_host=args.momentum_host, fp8_steps=args.fp8_steps)
    else:
        X = [d["x"] for d in ins]
        OUT = [torch.empty_like(x) for x in X]

        def step():
            nsa.ns_batched(X, steps=wl.steps, coeffs=wl.coeffs, eps=wl.eps, out=OUT, workspace=ws,
                           fp8_steps=args.fp8_steps)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # the headline: K steps, no per-kernel instrumentation
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize(dev)
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)
    # per-kernel durations: another K steps with HIP events around every launch
    nsa.timing_reset()
    nsa.timing_enable(True)
    torch.cuda.synchronize(dev)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize(dev)
    nsa.timing_enable(False)
    kern = nsa.timing_read()
    instrumented_ms = t_start.elapsed_time(t_end) / args.steps
    print(f"[bench] per-kernel pass: {instrumented_ms:.3f} ms/step with per-launch events",
          file=sys.stderr, flush=True)

    esize = 2 if wl.dtype == "bf16" else 4
    fl = [ns_flops(s, wl.steps, c != 0.0) for s in shapes]
    alg_total = sum(f[0] for f in fl)
    alg_prod_launch = sum(2 * min(s) ** 2 * max(s) for s in shapes)
    alg_gram_launch = sum(min(s) * (min(s) + 1) * max(s) for s in shapes)
    alg_poly_launch = sum(min(s) ** 2 * (min(s) + 1) for s in shapes)
    peak = PEAK_TFLOPS[wl.dtype]

    # with the momentum in host memory the step runs in chunks, one launch of
    # each kernel per chunk, so a launch covers 1/nchunks of the batch's work
    nchunks = max(1, round(kern["prepare"][1] / args.steps)) if args.momentum_host else 1

    def avg(name):
        ms, n = kern[name]
        return ms * nchunks / n if n else float("nan")

    # the middle products (the first takes the norm factor, the last the update)
    prod_ms = avg("prod") if kern["prod"][1] else avg("prod_first")
    achieved = alg_prod_launch / (prod_ms * 1e-3) / 1e12
    # avg_ms: per launch over the whole batch (the sum over a step's chunks)
    per_kernel = {k: {"avg_ms": round(avg(k), 4), "launches": kern[k][1]} for k in nsa.KERNELS
                  if kern[k][1]}
    ns_ms = sum(kern[k][0] for k in ("gram", "poly", "prod_first", "prod", "prod_finish", "quant8",
                                     "gram8", "poly8", "prod8")) / args.steps
    ew = [elementwise_bytes(s, esize, wl.call) for s in shapes]
    for name, idx in (("prepare", 0), ("finish", 1)):
        if name not in per_kernel:
            continue
        b = sum(e[idx] for e in ew)
        per_kernel[name]["gbs"] = round(b / (avg(name) * 1e-3) / 1e9, 1)
        per_kernel[name]["hbm_frac"] = round(b / (avg(name) * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)
    for name, flops in (("gram", alg_gram_launch), ("poly", alg_poly_launch), ("prod", alg_prod_launch),
                        ("prod_first", alg_prod_launch), ("gram8", alg_gram_launch),
                        ("poly8", alg_poly_launch), ("prod8", alg_prod_launch)):
        if kern[name][1]:
            t = flops / (avg(name) * 1e-3) / 1e12
            per_kernel[name]["tflops"] = round(t, 1)
            per_kernel[name]["mfma_frac"] = round(t / (PEAK_TFLOPS["e4m3"] if name.endswith("8")
                                                       else peak), 3)

    value = wl.batch * args.steps / (total_ms * 1e-3)
    metric = METRIC if args.fp8_steps == 0 else (
        METRIC + f" [e4m3 operands in the first {args.fp8_steps} NS steps]")
    result = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype if args.fp8_steps == 0 else wl.dtype + "+e4m3",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "shapes": sorted({tuple(s) for s in shapes}),
                   "ns_steps": wl.steps, "coeffs": list(wl.coeffs), "call": wl.call,
                   "nesterov": wl.nesterov, "lr": wl.lr, "beta": wl.beta,
                   "momentum": "pinned host memory" if args.momentum_host else "HBM",
                   "fp8_steps": args.fp8_steps},
        "roofline": {"bound": "mfma", "kernel": "prod (X <- aX + BX)", "achieved": round(achieved, 1),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": rocprof_summary.read_traffic(TRAFFIC_SUMMARY, wl.name)
                     if wl.name == TRAFFIC_WORKLOAD else None},
        "ns_effective_tflops": round(alg_total / (total_ms / args.steps * 1e-3) / 1e12, 1),
        "ns_mfma_frac_whole_step": round(alg_total / (total_ms / args.steps * 1e-3) / 1e12 / peak, 4),
        "ns_kernels_ms_per_step": round(ns_ms, 3),
        "per_kernel_pass_ms_per_step": round(instrumented_ms, 3),
        "kernels": per_kernel,
    }
    if args.momentum_host:
        # the DMA copies, timed by the library on its copy streams: how much of
        # them the step hides behind the Newton-Schulz kernels
        in_ms, out_ms = kern["mom_in"][0] / args.steps, kern["mom_out"][0] / args.steps
        gpu_ms = sum(kern[k][0] for k in nsa.KERNELS if not k.startswith("mom_")) / args.steps
        mbytes = sum(esize * r * c for r, c in shapes)
        result["momentum_chunks"] = nchunks
        result["momentum_copies"] = {
            "to_device_ms_per_step": round(in_ms, 3), "to_host_ms_per_step": round(out_ms, 3),
            "to_device_gbs": round(mbytes / (in_ms * 1e-3) / 1e9, 1),
            "to_host_gbs": round(mbytes / (out_ms * 1e-3) / 1e9, 1),
            "kernels_ms_per_step": round(gpu_ms, 3),
            "serial_ms_per_step": round(in_ms + out_ms + gpu_ms, 3),
            "measured_ms_per_step": round(instrumented_ms, 3)}
    if (not args.no_variants and wl.call == "step" and wl.dtype == "bf16" and not args.momentum_host
            and args.fp8_steps == 0):
        result["variants"] = bench_variants(args, wl, W, G, M, shapes, dev)
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
