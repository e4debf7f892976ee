"""Helpers shared by the GPU parity tests: inputs, metrics and tolerances.

Tolerances (relative Frobenius error of the HIP result against the float64
oracle on the same dtype-cast inputs): 2e-2 for bf16 storage with fp32
matrix-core accumulation, 1e-4 for the fp32 mode.

The bf16 tolerance is applied to every 256 x 256 block of a result, not only
to the whole matrix: the matrix-core kernels work in 256 x 256 output tiles,
so a mistake confined to one tile (an index, a mirror store, a term dropped
on one tile) shows in that block at full size, where in a 2048 x 6144
matrix it would move the whole-matrix figure by about 1/14 of its size.  The
bf16 error of a correct run is spread evenly over the blocks (it comes from
the roundings of the iterate, A and B, which act on the whole spectrum), so
the per-block gate keeps the same headroom as the whole-matrix one.
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


BLOCK = 256          # the matrix-core output tile
MIN_EDGE = 64        # a last piece thinner than this joins its neighbour


def block_cuts(n: int, block: int = BLOCK, min_edge: int = MIN_EDGE):
    """Edges of the pieces of a side of length n: multiples of `block`, with a
    last piece thinner than `min_edge` merged into the one before it."""
    cuts = list(range(0, n, block)) + [n]
    if len(cuts) > 2 and cuts[-1] - cuts[-2] < min_edge:
        del cuts[-2]
    return cuts


def block_errors(got, want, block: int = BLOCK, min_edge: int = MIN_EDGE) -> np.ndarray:
    """Relative Frobenius error of every block (rows x cols grid of pieces)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    rc, cc = block_cuts(got.shape[0], block, min_edge), block_cuts(got.shape[1], block, min_edge)
    out = np.zeros((len(rc) - 1, len(cc) - 1))
    for i in range(len(rc) - 1):
        for j in range(len(cc) - 1):
            g = got[rc[i]:rc[i + 1], cc[j]:cc[j + 1]]
            w = want[rc[i]:rc[i + 1], cc[j]:cc[j + 1]]
            n = np.linalg.norm(w)
            out[i, j] = np.linalg.norm(g - w) / (n if n > 0 else 1.0)
    return out


def check_blocks(got, want, tol: float, what="") -> float:
    """Asserts that every block of `got` is within `tol` of `want`; returns the worst."""
    errs = block_errors(got, want)
    worst = float(errs.max())
    if worst > tol:
        i, j = np.unravel_index(int(np.argmax(errs)), errs.shape)
        raise AssertionError(f"{what}: block ({i}, {j}) of {errs.shape} has relative error "
                             f"{worst:.3e} > {tol:.1e} (whole matrix {rel_fro(got, want):.3e})")
    return worst


def momentum_within_rounding(m0, g, m1, beta: float, dtype: str):
    """M' = beta*M + G stored in the dtype: half an ulp of the exact value, plus the
    fp32 evaluation of beta*M + G relative to its operands.  Arrays are float64
    copies of the dtype values; returns the boolean mask of violations."""
    m0, g, m1 = (np.asarray(t, np.float64) for t in (m0, g, m1))
    want = beta * m0 + g
    ulp = np.spacing(np.maximum(np.abs(want), np.abs(m1)).astype(np.float32)).astype(np.float64)
    if dtype == "bf16":
        ulp *= 2.0 ** 16
    bound = 0.5 * ulp + 4.0 * 2.0 ** -24 * (beta * np.abs(m0) + np.abs(g))
    return np.abs(m1 - want) > bound * (1 + 1e-12)


def update_step(rows: int, cols: int, lr: float) -> float:
    """lr * sqrt(max(1, rows/cols)): the factor of O in the weight update."""
    return lr * float(np.sqrt(max(1.0, rows / cols)))


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
