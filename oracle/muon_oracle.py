"""Plain float64 CPU oracle of the batched Muon step.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module.  The HIP library never links, calls
or reads anything here, and nothing here comes from the HIP path.

What is computed, and where it comes from:

* Muon keeps a single optimizer state per weight matrix ("Domyn is training a
  1T-parameter MoE on Europe's Jupiter supercomputer, and published the
  recipe", §What moved the number, Longer sequences bullet).  The reading taken
  here is heavy-ball momentum without dampening, M' = beta*M + G, with the
  Nesterov variant U = G + beta*M'; otherwise U = M'.
* The Newton-Schulz update works on whole matrices ("How PyTorch Scaled a
  Near-1T MoE on Europe's Public Supercomputer", §Three optimizations that
  changed the economics, FlexShard bullet).  The pages fix no polynomial; the
  reading taken is the odd polynomial iteration on the short side:
  X0 = U / (||U||_F + eps);  repeat k times:  A = X X^T,  B = b A + c A A,
  X = a X + B X;  with U transposed first when it has more rows than columns.
* The weight update is W' = W - lr * sqrt(max(1, rows/cols)) * O, with rows
  and cols those of the stored matrix.

Every step is written out in the order above in float64 numpy, with numpy's
matrix product as the only library primitive.  No blocking, fusion or
reordering.  Inputs are expected to be the exact float64 upcast of the
dtype-cast values the GPU sees.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np

QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)
DEFAULT_EPS = 1e-7


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def momentum(m, g, beta: float) -> np.ndarray:
    """New momentum buffer M' = beta*M + G (the single optimizer state)."""
    return beta * _f64(m) + _f64(g)


def nesterov_direction(g, m_new, beta: float) -> np.ndarray:
    """Nesterov look-ahead direction U = G + beta*M', using the new buffer."""
    return _f64(g) + beta * _f64(m_new)


def frobenius_norm(u) -> float:
    """||U||_F = sqrt of the sum of squared entries."""
    u = _f64(u)
    return math.sqrt(float(np.sum(u * u)))


def is_tall(rows: int, cols: int) -> bool:
    """Tall matrices (more rows than columns) are orthogonalized as their transpose."""
    return rows > cols


def normalize(u, eps: float = DEFAULT_EPS) -> np.ndarray:
    """X0 = U / (||U||_F + eps)."""
    u = _f64(u)
    return u / (frobenius_norm(u) + eps)


def newton_schulz(u, steps: int, coeffs: Sequence[float] = QUINTIC,
                  eps: float = DEFAULT_EPS) -> np.ndarray:
    """k Newton-Schulz iterations on the short side of U; output has U's shape.

    X0 = U/(||U||_F+eps) in the wide orientation; each iteration forms the
    Gram matrix A = X X^T of the short side, the polynomial B = bA + cA^2, and
    multiplies back X <- aX + BX.
    """
    a, b, c = (float(t) for t in coeffs)
    u = _f64(u)
    tall = is_tall(*u.shape)
    x = normalize(u.T if tall else u, eps)
    for _ in range(steps):
        gram = x @ x.T
        poly = b * gram + c * (gram @ gram)
        x = a * x + poly @ x
    return x.T if tall else x


def update_scale(rows: int, cols: int) -> float:
    """Shape-dependent scale of the orthogonalized update, sqrt(max(1, rows/cols))."""
    return math.sqrt(max(1.0, rows / cols))


def apply_update(w, o, lr: float) -> np.ndarray:
    """W' = W - lr * sqrt(max(1, rows/cols)) * O."""
    w = _f64(w)
    rows, cols = w.shape
    return w - lr * update_scale(rows, cols) * _f64(o)


def muon_step(w, g, m, lr: float = 0.02, beta: float = 0.95, nesterov: bool = False,
              steps: int = 5, coeffs: Sequence[float] = QUINTIC,
              eps: float = DEFAULT_EPS) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One Muon step on one matrix. Returns (W', M', O)."""
    m_new = momentum(m, g, beta)
    u = nesterov_direction(g, m_new, beta) if nesterov else m_new
    o = newton_schulz(u, steps, coeffs, eps)
    return apply_update(w, o, lr), m_new, o

