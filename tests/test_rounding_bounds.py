"""CPU checks of the elementwise rounding bound (tests/rounding_bounds.py).

The bound is what the GPU parity tests hold every bf16 output element to, so
it is pinned here against things other than itself:

- its exact iteration equals the oracle's result;
- a bf16 emulation of the library's rounding points (fp32 products, bf16
  stores of A, B and X, the norm factor applied as the first Gram and product
  store) stays within it;
- the same emulation with a planted mistake (a dropped a X term, or the norm
  factor applied once instead of squared in the first Gram) leaves it by a wide
  margin, so the bound is tight enough to catch such mistakes.
"""
import numpy as np
import pytest
import torch

import oracle
from rounding_bounds import ns_with_bound

SHAPES = [(64, 160), (160, 64), (97, 300)]
CASES = [((0.0, 1.0, 0.0), 1), ((0.0, 0.0, 1.0), 1), ((0.5, 0.25, 0.125), 2), ((1.0, 0.0, 0.0), 2),
         ((0.5, 0.25, 0.125), 3)]


def _rb(t):
    """fp32 -> bf16 (round to nearest even) -> fp32."""
    return t.to(torch.bfloat16).to(torch.float32)


def _emulate(u, steps, coeffs, mistake=None, eps=1e-7):
    """The iteration at the library's rounding points on the bf16 input u."""
    a, b, c = coeffs
    u = torch.as_tensor(u, dtype=torch.float32)
    tall = u.shape[0] > u.shape[1]
    x = _rb(u.T.contiguous() if tall else u)
    f = 1.0 / (float(torch.linalg.norm(x.double())) + eps)
    for k in range(steps):
        first = k == 0
        g = (f if mistake == "norm_once" else f * f) if first else 1.0
        A = _rb((x @ x.T) * (g * (1.0 if c != 0 else b)))
        B = _rb(c * (A @ A + (b / c) * A)) if c != 0 else A
        t = B @ x if mistake == "no_ax" else a * x + B @ x
        x = _rb(t * (f if first else 1.0))
    return (x.T if tall else x).double().numpy()


def _input(shape, seed):
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))
    return x.to(torch.bfloat16).to(torch.float32)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("coeffs,steps", CASES)
def test_bound_holds_for_the_rounding_points(shape, coeffs, steps):
    x = _input(shape, 3)
    u = x.double().numpy()
    exact, bound = ns_with_bound(u, steps, coeffs)
    want = oracle.newton_schulz(u, steps, coeffs)
    assert np.max(np.abs(exact - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))
    ratio = np.max(np.abs(_emulate(x, steps, coeffs) - exact) / bound)
    assert ratio <= 1.0, ratio


@pytest.mark.parametrize("mistake,coeffs,steps", [("no_ax", (1.0, 0.0, 0.0), 2),
                                                  ("no_ax", (0.5, 0.25, 0.125), 2),
                                                  ("norm_once", (0.0, 1.0, 0.0), 1),
                                                  ("norm_once", (0.5, 0.25, 0.125), 2)])
def test_planted_mistakes_leave_the_bound(mistake, coeffs, steps):
    x = _input((97, 300), 4)
    exact, bound = ns_with_bound(x.double().numpy(), steps, coeffs)
    ratio = np.max(np.abs(_emulate(x, steps, coeffs, mistake) - exact) / bound)
    assert ratio > 10, ratio
