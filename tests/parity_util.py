"""Helpers shared by the GPU parity tests: inputs, metrics and tolerances.

Tolerances (relative Frobenius error of the HIP result against the float64
oracle on the same dtype-cast inputs): 2e-2 for bf16 storage with fp32
matrix-core accumulation, 1e-4 for the fp32 mode.
"""
from __future__ import annotations

import concurrent.futures
import os

import numpy as np

import workloads

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def rel_fro(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    n = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (n if n > 0 else 1.0))


def torch_dtype(name: str):
    import torch

    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def _host_inputs(wl, j):
    raw = workloads.matrix_inputs(wl, j)
    return {k: workloads.cast(v, wl.dtype) for k, v in raw.items()}


def device_inputs(wl, device="cuda", indices=None, threads=None):
    """Per-matrix dicts of device tensors (cast on the host, then copied)."""
    import torch

    idx = list(range(wl.batch)) if indices is None else list(indices)
    threads = threads or min(16, os.cpu_count() or 1)
    out = [None] * len(idx)
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        futs = {ex.submit(_host_inputs, wl, j): n for n, j in enumerate(idx)}
        for f in concurrent.futures.as_completed(futs):
            n = futs[f]
            out[n] = {k: v.to(device, non_blocking=False) for k, v in f.result().items()}
    torch.cuda.synchronize()
    return out


def host_f64(t) -> np.ndarray:
    return workloads.as_float64(t)


def singular_values(a) -> np.ndarray:
    return np.linalg.svd(np.asarray(a, np.float64), compute_uv=False)
