"""Pins of the CPU oracle against facts that do not come from the oracle.

* closed form: any odd polynomial iteration acts on singular values only, so
  NS_k(X) = U f_k(S / (||X||_F + eps)) V^T with f_k the k-fold scalar map
  p(x) = a x + b x^3 + c x^5, computed here from LAPACK's SVD;
* the cubic (1.5, -0.5) iteration converges to the polar factor U V^T
  (scipy.linalg.polar);
* orthogonal invariance NS(Q X R) = Q NS(X) R and transpose invariance;
* the singular-value band of the quintic iteration;
* special cases (zero input, one row, orthonormal rows, steps = 0);
* the momentum buffer equals torch.optim.SGD's (dampening 0, with and without
  Nesterov);
* the update scale sqrt(max(1, rows/cols)) on hand-computed values.

The last test plants plausible mistakes in copies of the oracle and checks
that every one of them fails at least one pin.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
import workloads

QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)


def scalar_map(x, steps, coeffs):
    a, b, c = coeffs
    x = np.array(x, dtype=np.float64)
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def svd_closed_form(x, steps, coeffs, eps=1e-7):
    x = np.asarray(x, np.float64)
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    f = scalar_map(s / (np.linalg.norm(x) + eps), steps, coeffs)
    return (u * f) @ vt


def rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def haar(n, rng):
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))


def c1_input():
    wl = workloads.standard_workloads()["c1_fp32_256x512"]
    return workloads.as_float64(workloads.cast(workloads.matrix_inputs(wl, 0)["x"], "fp32"))


# --------------------------------------------------------------------------
# Pins as predicates, so that the same checks can be run on planted mistakes.
# --------------------------------------------------------------------------

def pin_closed_form(ns):
    rng = np.random.default_rng(10)
    worst = 0.0
    for shape in [(24, 40), (40, 24), (33, 33), (5, 61)]:
        x = rng.standard_normal(shape)
        for steps, coeffs in [(5, QUINTIC), (3, CUBIC), (2, (2.0, -1.5, 0.5))]:
            worst = max(worst, rel(ns(x, steps, coeffs), svd_closed_form(x, steps, coeffs)))
    return worst < 1e-12, worst


def pin_polar(ns):
    x = c1_input()
    polar_u, _ = scipy.linalg.polar(x)
    err = rel(ns(x, 30, CUBIC), polar_u)
    return err < 1e-10, err


def pin_orthogonal_invariance(ns):
    rng = np.random.default_rng(11)
    worst = 0.0
    for m, n in [(20, 36), (36, 20)]:
        x = rng.standard_normal((m, n))
        q, r = haar(m, rng), haar(n, rng)
        worst = max(worst, rel(ns(q @ x @ r, 5, QUINTIC), q @ ns(x, 5, QUINTIC) @ r))
    return worst < 1e-12, worst


def pin_band(ns):
    """Quintic, 5 steps: outputs of the 256x512 workload lie in the scalar map's band."""
    x = c1_input()
    sv_in = np.linalg.svd(x, compute_uv=False) / (np.linalg.norm(x) + 1e-7)
    grid = np.geomspace(sv_in.min(), 1.0, 200001)
    f = scalar_map(grid, 5, QUINTIC)
    sv_out = np.linalg.svd(ns(x, 5, QUINTIC), compute_uv=False)
    ok = (sv_out.min() >= f.min() - 1e-9) and (sv_out.max() <= f.max() + 1e-9)
    # the band derived for inputs with normalized sigma >= 5.18e-3
    ok = ok and sv_in.min() >= 5.18e-3 and 0.6818 <= sv_out.min() and sv_out.max() <= 1.1344
    return ok, (sv_out.min(), sv_out.max())


def pin_special_cases(ns):
    errs = []
    errs.append(float(np.abs(ns(np.zeros((7, 11)), 5, QUINTIC)).max()))
    x = np.arange(1.0, 10.0).reshape(1, 9)
    nx = math.sqrt(float(np.sum(x * x)))
    want = x / nx * scalar_map(nx / (nx + 1e-7), 5, QUINTIC)
    errs.append(rel(ns(x, 5, QUINTIC), want))
    rng = np.random.default_rng(12)
    q = haar(16, rng)[:6]  # 6 x 16, orthonormal rows
    want = scalar_map(1.0 / (math.sqrt(6.0) + 1e-7), 5, QUINTIC) * q  # sigma = 1/||q||_F
    errs.append(rel(ns(q, 5, QUINTIC), want))
    y = rng.standard_normal((9, 4))
    errs.append(rel(ns(y, 0, QUINTIC), y / (np.linalg.norm(y) + 1e-7)))
    return max(errs) < 1e-12, errs


def pin_transpose(ns):
    rng = np.random.default_rng(13)
    x = rng.standard_normal((12, 30))
    exact = np.array_equal(ns(x.T, 5, QUINTIC), ns(x, 5, QUINTIC).T)
    sq = rng.standard_normal((17, 17))
    return exact and rel(ns(sq.T, 5, QUINTIC), ns(sq, 5, QUINTIC).T) < 1e-12, exact


def sgd_reference(w, g, m, lr, beta, nesterov):
    """torch.optim.SGD (dampening 0) on CPU: returns (new buffer, direction)."""
    p = torch.nn.Parameter(torch.from_numpy(w.copy()))
    opt = torch.optim.SGD([p], lr=lr, momentum=beta, dampening=0.0, nesterov=nesterov)
    p.grad = torch.from_numpy(g.copy())
    opt.state[p]["momentum_buffer"] = torch.from_numpy(m.copy())
    opt.step()
    buf = opt.state[p]["momentum_buffer"].numpy().copy()
    direction = (w - p.detach().numpy()) / lr
    return buf, direction


def pin_momentum(momentum, direction):
    rng = np.random.default_rng(14)
    w, g, m = (rng.standard_normal((6, 10)) for _ in range(3))
    worst = 0.0
    for nesterov in (False, True):
        buf, d = sgd_reference(w, g, m, 0.5, 0.95, nesterov)
        m_new = momentum(m, g, 0.95)
        worst = max(worst, rel(m_new, buf), rel(direction(g, m_new, 0.95, nesterov), d))
    return worst < 1e-12, worst


def oracle_direction(g, m_new, beta, nesterov):
    return oracle.nesterov_direction(g, m_new, beta) if nesterov else m_new


def pin_update_scale(scale):
    cases = {(6144, 2048): math.sqrt(3.0), (2048, 6144): 1.0, (3, 1): math.sqrt(3.0),
             (1024, 1024): 1.0, (6144, 1024): math.sqrt(6.0)}
    worst = max(abs(scale(*k) - v) for k, v in cases.items())
    return worst < 1e-15, worst


def ns_oracle(x, steps, coeffs):
    return oracle.newton_schulz(x, steps, coeffs)


# --------------------------------------------------------------------------
# The oracle against its pins.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("pin", [pin_closed_form, pin_polar, pin_orthogonal_invariance,
                                 pin_band, pin_special_cases, pin_transpose])
def test_ns_pin(pin):
    ok, detail = pin(ns_oracle)
    assert ok, detail


def test_momentum_matches_torch_sgd():
    ok, detail = pin_momentum(oracle.momentum, oracle_direction)
    assert ok, detail


def test_update_scale_hand_values():
    ok, detail = pin_update_scale(oracle.update_scale)
    assert ok, detail
    w = np.zeros((6, 2))
    assert np.allclose(oracle.apply_update(w, np.ones((6, 2)), 0.02), -0.02 * math.sqrt(3.0))


def test_full_step_composition():
    """W', M', O of one step, against SGD's buffer, the SVD closed form and the scale."""
    rng = np.random.default_rng(15)
    for (rows, cols), nesterov in [((10, 26), False), ((26, 10), True)]:
        w, g, m = (rng.standard_normal((rows, cols)) for _ in range(3))
        w2, m2, o = oracle.muon_step(w, g, m, lr=0.02, beta=0.95, nesterov=nesterov, steps=5)
        buf, d = sgd_reference(w, g, m, 0.02, 0.95, nesterov)
        assert rel(m2, buf) < 1e-12
        want_o = svd_closed_form(d, 5, QUINTIC)
        assert rel(o, want_o) < 1e-12
        scale = math.sqrt(max(1.0, rows / cols))
        assert np.abs(w2 - (w - 0.02 * scale * want_o)).max() < 1e-12


def test_scale_invariance():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((20, 30))
    # exact in the absence of eps; eps/||x|| ~ 4e-9 shifts the normalized spectrum,
    # and the quintic map's slope (at most a^5 ~ 486) amplifies that shift
    assert rel(oracle.newton_schulz(1e3 * x, 5), oracle.newton_schulz(x, 5)) < 1e-5
    assert rel(oracle.newton_schulz(1e3 * x, 5, eps=0.0), oracle.newton_schulz(x, 5, eps=0.0)) < 1e-12


def test_default_coefficients():
    """Defaults are the quintic (3.4445, -4.7750, 2.0315) and cubic (1.5, -0.5, 0)."""
    assert oracle.QUINTIC == (3.4445, -4.7750, 2.0315)
    assert oracle.CUBIC == (1.5, -0.5, 0.0)
    assert workloads.QUINTIC == oracle.QUINTIC and workloads.CUBIC == oracle.CUBIC


# --------------------------------------------------------------------------
# Planted mistakes (copies of the oracle on the CPU): each must fail a pin.
# --------------------------------------------------------------------------

def _ns_mutant(kind):
    def ns(x, steps, coeffs, eps=1e-7):
        a, b, c = coeffs
        x = np.asarray(x, np.float64)
        tall = x.shape[0] > x.shape[1]
        if kind == "no_transpose_back":
            x = x.T if tall else x
            tall = False
        else:
            x = x.T if tall else x
        if kind == "spectral_norm":
            x = x / (np.linalg.norm(x, 2) + eps)
        elif kind == "eps_in_sqrt":
            x = x / math.sqrt(float(np.sum(x * x)) + eps)
        elif kind == "no_normalize":
            pass
        else:
            x = x / (np.linalg.norm(x) + eps)
        for _ in range(steps):
            g = x @ x.T
            if kind == "drop_c":
                p = b * g
            elif kind == "sign_b":
                p = -b * g + c * (g @ g)
            elif kind == "c_times_a_only":
                p = b * g + c * g
            else:
                p = b * g + c * (g @ g)
            if kind == "drop_a":
                x = p @ x
            elif kind == "swap_ab":
                x = b * x + (a * g + c * (g @ g)) @ x
            else:
                x = a * x + p @ x
        return x.T if tall else x
    return ns


NS_MUTANTS = ["no_transpose_back", "spectral_norm", "no_normalize", "drop_c", "sign_b",
              "c_times_a_only", "drop_a", "swap_ab", "eps_in_sqrt"]


@pytest.mark.parametrize("kind", NS_MUTANTS)
def test_planted_ns_mistake_fails_a_pin(kind):
    ns = _ns_mutant(kind)
    results = []
    for pin in [pin_closed_form, pin_polar, pin_orthogonal_invariance, pin_band,
                pin_special_cases, pin_transpose]:
        try:
            ok, _ = pin(ns)
        except (ValueError, FloatingPointError):  # a shape error also counts as caught
            ok = False
        results.append(ok)
    assert not all(results), f"mutant {kind} passed every pin"


def test_planted_momentum_mistakes_fail_a_pin():
    mutants = [
        (lambda m, g, beta: beta * m + (1 - beta) * g, oracle_direction),  # dampening
        (lambda m, g, beta: m + beta * g, oracle_direction),  # swapped roles
        (oracle.momentum, lambda g, m_new, beta, nesterov:  # Nesterov with the old buffer
            g + beta * (m_new - g) / beta if nesterov else m_new),
    ]
    for mom, direction in mutants:
        ok, _ = pin_momentum(mom, direction)
        assert not ok
    ok, _ = pin_update_scale(lambda r, c: math.sqrt(max(1.0, c / r)))
    assert not ok
