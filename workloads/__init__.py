"""Seeded synthetic inputs for the batched Muon step.

This module holds the shapes, value distributions and seeds of the workloads
and nothing of the step's arithmetic.  Both the HIP path (through its tests and
bench.py) and the CPU oracle are fed from here, so the two sides see the same
bits.

Shapes follow the model described on "How PyTorch Scaled a Near-1T MoE on
Europe's Public Supercomputer", §Introduction (74 layers, 384 routed experts,
hidden size 6,144) and the FlexShard bullet of §Three optimizations that
changed the economics (whole experts placed on one rank).  The expert FFN
width of 2048 is an assumption: the pages give only the hidden size.

Random streams: every (workload seed, matrix index, tensor id) triple gets its
own numpy PCG64 stream, ``numpy.random.default_rng([seed, j, tid])``.  A
matrix can therefore be regenerated alone, which is what lets a full-size
batch be checked against the oracle on sampled matrices.  Values are drawn in
float32 and cast to the working dtype by torch on the CPU, which rounds to
nearest even.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Sequence, Tuple

import numpy as np

# Tensor ids inside a matrix's stream family.
_TID_W, _TID_M, _TID_G, _TID_X = 1, 2, 3, 4
_TID_U, _TID_V, _TID_S = 5, 6, 7
_TID_SHAPES = 99

QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)

EXPERT_SHAPES = {"gate": (6144, 2048), "up": (6144, 2048), "down": (2048, 6144)}
MIXED_DIMS = (512, 1024, 2048, 6144)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: a ragged batch of matrices plus step settings.

    kind:
      "gauss"   - X ~ N(0, 1) (input of the orthogonalization alone);
      "muon"    - W ~ N(0, 0.02^2), M ~ N(0, std_m^2), G ~ N(0, std_g^2);
      "illcond" - W ~ N(0, 0.02^2), M = 0, G = U diag(s) V^T with s
                  log-uniform on [1e-4, 1] and U, V with orthonormal columns.
    """

    name: str
    dtype: str  # "bf16" or "fp32"
    shapes: Tuple[Tuple[int, int], ...]
    call: str  # "ns" or "step"
    kind: str
    steps: int = 5
    coeffs: Tuple[float, float, float] = QUINTIC
    eps: float = 1e-7
    lr: float = 0.02
    beta: float = 0.95
    nesterov: bool = False
    std_w: float = 0.02
    std_m: float = 1e-3
    std_g: float = 1e-3
    seed: int = 0

    @property
    def batch(self) -> int:
        return len(self.shapes)

    def with_shapes(self, shapes: Sequence[Tuple[int, int]], name: str | None = None) -> "Workload":
        return dataclasses.replace(self, shapes=tuple(tuple(s) for s in shapes),
                                   name=name or self.name)


def _mixed_shapes(seed: int, count: int) -> Tuple[Tuple[int, int], ...]:
    rng = np.random.default_rng([seed, _TID_SHAPES])
    dims = rng.choice(np.array(MIXED_DIMS), size=(count, 2))
    return tuple((int(r), int(c)) for r, c in dims)


def _one_rank_expert_shapes(layers: int = 74) -> Tuple[Tuple[int, int], ...]:
    out: List[Tuple[int, int]] = []
    for _ in range(layers):
        out += [EXPERT_SHAPES["gate"], EXPERT_SHAPES["up"], EXPERT_SHAPES["down"]]
    return tuple(out)


def standard_workloads() -> Dict[str, Workload]:
    """The five standard workloads, at full size."""
    return {
        "c1_fp32_256x512": Workload(
            name="c1_fp32_256x512", dtype="fp32", shapes=((256, 512),), call="ns",
            kind="gauss", steps=5, seed=1),
        "c2_96x2048x6144": Workload(
            name="c2_96x2048x6144", dtype="bf16", shapes=((2048, 6144),) * 96, call="step",
            kind="muon", steps=5, seed=2),
        "c3_rank_222_experts": Workload(
            name="c3_rank_222_experts", dtype="bf16", shapes=_one_rank_expert_shapes(), call="step",
            kind="muon", steps=5, seed=3),
        "c4_dense_attn": Workload(
            name="c4_dense_attn", dtype="bf16",
            shapes=((6144, 6144),) * 16 + ((6144, 1024),) * 16, call="ns",
            kind="gauss", steps=5, seed=4),
        "c5_mixed_illcond": Workload(
            name="c5_mixed_illcond", dtype="bf16", shapes=_mixed_shapes(5, 128), call="step",
            kind="illcond", steps=10, nesterov=True, seed=5),
    }


@dataclasses.dataclass(frozen=True)
class AdamWWorkload:
    """A ragged batch of flat tensors for the AdamW step.

    p ~ N(0, std_p^2), g ~ N(0, std_g^2), m ~ N(0, std_m^2), v = (N(0, std_m))^2
    (non-negative, as a second moment is); p and g in `dtype`, m and v fp32.
    """

    name: str
    dtype: str
    numels: Tuple[int, ...]
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    step: int = 10
    std_p: float = 0.02
    std_g: float = 1e-3
    std_m: float = 1e-3
    seed: int = 6

    @property
    def batch(self) -> int:
        return len(self.numels)


HIDDEN = 6144
LAYERS = 74
ROUTED_EXPERTS = 384


def adamw_workloads() -> Dict[str, AdamWWorkload]:
    """The non-expert parameters of the model, for AdamW: per layer two norm
    weights (hidden size) and the router (routed experts x hidden), plus the
    final norm; 175.5 M elements in 223 tensors."""
    numels: List[int] = []
    for _ in range(LAYERS):
        numels += [HIDDEN, HIDDEN, ROUTED_EXPERTS * HIDDEN]
    numels.append(HIDDEN)
    return {
        "adamw_nonexpert_74_layers": AdamWWorkload(
            name="adamw_nonexpert_74_layers", dtype="bf16", numels=tuple(numels)),
    }


def adamw_inputs(wl: AdamWWorkload, j: int) -> Dict[str, np.ndarray]:
    """Inputs of tensor j as float32 arrays (p and g before the dtype cast)."""
    n = wl.numels[j]
    m = _normal(wl.seed, j, _TID_M, (n,), wl.std_m)
    v = _normal(wl.seed, j, _TID_V, (n,), wl.std_m)
    return {"p": _normal(wl.seed, j, _TID_W, (n,), wl.std_p),
            "g": _normal(wl.seed, j, _TID_G, (n,), wl.std_g),
            "m": m, "v": v * v}


def c1_cubic() -> Workload:
    """Workload 1 in its cubic mode: (a, b, c) = (1.5, -0.5, 0), 30 steps."""
    return dataclasses.replace(standard_workloads()["c1_fp32_256x512"],
                               name="c1_fp32_256x512_cubic30", coeffs=CUBIC, steps=30)


# ---------------------------------------------------------------------------
# Per-matrix generation (float32 numpy arrays; cast with `cast`).
# ---------------------------------------------------------------------------

def _normal(seed: int, j: int, tid: int, shape, std: float) -> np.ndarray:
    rng = np.random.default_rng([seed, j, tid])
    out = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _orthonormal_columns(seed: int, j: int, tid: int, rows: int, k: int) -> np.ndarray:
    """rows x k matrix with orthonormal columns: Q of a Gaussian, signs of diag(R) fixed."""
    g = _normal(seed, j, tid, (rows, k), 1.0).astype(np.float64)
    q, r = np.linalg.qr(g)
    d = np.sign(np.diag(r))
    d[d == 0] = 1.0
    return q * d


def illcond_spectrum(seed: int, j: int, k: int) -> np.ndarray:
    """k singular values, log-uniform on [1e-4, 1]."""
    rng = np.random.default_rng([seed, j, _TID_S])
    return 10.0 ** rng.uniform(-4.0, 0.0, size=k)


def illcond_factors(wl: Workload, j: int):
    """(U, s, V) with G_j = U diag(s) V^T before the float32 rounding (kind "illcond")."""
    rows, cols = wl.shapes[j]
    k = min(rows, cols)
    u = _orthonormal_columns(wl.seed, j, _TID_U, rows, k)
    v = _orthonormal_columns(wl.seed, j, _TID_V, cols, k)
    return u, illcond_spectrum(wl.seed, j, k), v


def illcond_inputs_device(wl: Workload, j: int, device):
    """Inputs of matrix j of an "illcond" workload, built on `device`.

    Same recipe as `matrix_inputs` (the same seeded float32 Gaussians, QR with
    the signs of diag(R) fixed, s log-uniform on [1e-4, 1]), with the QR and
    U diag(s) V^T done in float64 on the device, which is much faster for
    6144-sided matrices.  The bits differ from the host version's, so a caller
    checks against the oracle by copying these tensors back.  Returns
    ({"w", "m", "g"} in the working dtype, (U, s, V) float64 on the device).
    """
    import torch

    rows, cols = wl.shapes[j]
    k = min(rows, cols)

    def ortho(tid, n):
        a = torch.from_numpy(_normal(wl.seed, j, tid, (n, k), 1.0)).to(device, torch.float64)
        q, r = torch.linalg.qr(a)
        d = torch.sign(torch.diagonal(r))
        d[d == 0] = 1.0
        return q * d

    u = ortho(_TID_U, rows)
    v = ortho(_TID_V, cols)
    s = torch.from_numpy(illcond_spectrum(wl.seed, j, k)).to(device, torch.float64)
    g = torch.matmul(u * s, v.t().contiguous()).to(torch.float32)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    w = cast(_normal(wl.seed, j, _TID_W, (rows, cols), wl.std_w), wl.dtype).to(device)
    ins = {"w": w, "m": torch.zeros((rows, cols), dtype=tdt, device=device), "g": g.to(tdt)}
    return ins, (u, s, v)


def matrix_inputs(wl: Workload, j: int) -> Dict[str, np.ndarray]:
    """Inputs of matrix j of workload `wl`, as float32 arrays before the dtype cast."""
    rows, cols = wl.shapes[j]
    if wl.kind == "gauss":
        return {"x": _normal(wl.seed, j, _TID_X, (rows, cols), 1.0)}
    w = _normal(wl.seed, j, _TID_W, (rows, cols), wl.std_w)
    if wl.kind == "muon":
        m = _normal(wl.seed, j, _TID_M, (rows, cols), wl.std_m)
        g = _normal(wl.seed, j, _TID_G, (rows, cols), wl.std_g)
        return {"w": w, "m": m, "g": g}
    if wl.kind == "illcond":
        u, s, v = illcond_factors(wl, j)
        g = ((u * s) @ v.T).astype(np.float32)
        return {"w": w, "m": np.zeros((rows, cols), np.float32), "g": g}
    raise ValueError(f"unknown workload kind {wl.kind!r}")


def cast(arr: np.ndarray, dtype: str):
    """Cast a float32 array to the working dtype (torch CPU tensor, RNE for bf16)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "fp32":
        return t.to(torch.float32)
    raise ValueError(dtype)


def as_float64(t) -> np.ndarray:
    """Exact float64 copy of a (CPU or device) tensor, for the oracle."""
    import torch

    return t.detach().to("cpu", torch.float64).numpy()
