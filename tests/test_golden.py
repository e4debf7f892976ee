"""Oracle against hand-derived closed forms stored under tests/golden/.

The pages print no worked Newton-Schulz example, so the fixtures hold
textbook closed forms of the polar factor, which the cubic iteration
(1.5, -0.5, 0) converges to.  Each fixture states its derivation.  Nothing in
a fixture comes from the oracle or from the HIP path.
"""
import math
import pathlib

import numpy as np
import pytest

import oracle

GOLDEN = pathlib.Path(__file__).parent / "golden"


def read_fixture(name):
    lines = [ln.strip() for ln in (GOLDEN / name).read_text().splitlines()
             if ln.strip() and not ln.lstrip().startswith("#")]
    head = lines[0].split()
    assert head[0] == "input"
    rows, cols = int(head[1]), int(head[2])
    m = np.array([[float(v) for v in ln.split()] for ln in lines[1:1 + rows]])
    assert m.shape == (rows, cols)
    kind = lines[1 + rows].split()
    body = lines[2 + rows:2 + 2 * rows]
    if kind[0] == "expected":
        k = int(kind[1][len("sqrt("):-1])
        want = np.array([[float(v) for v in ln.split()] for ln in body]) / math.sqrt(k)
    else:
        assert kind[0] == "expected_expr"
        r = math.sqrt(80.0)
        t = math.sqrt(25.0 + 2.0 * r)
        want = np.array([[eval(e, {}, {"r": r, "t": t}) for e in ln.split()] for ln in body])
    return m, want


@pytest.mark.parametrize("name", ["polar_2x2.txt", "polar_wide_2x3.txt"])
def test_cubic_reaches_closed_form_polar_factor(name):
    m, want = read_fixture(name)
    # the factor itself is orthogonal / has orthonormal rows
    np.testing.assert_allclose(want @ want.T, np.eye(m.shape[0]), atol=1e-14)
    got = oracle.newton_schulz(m, 30, oracle.CUBIC, eps=0.0)
    np.testing.assert_allclose(got, want, atol=1e-13)
    # and the tall orientation gives the transpose
    got_t = oracle.newton_schulz(m.T, 30, oracle.CUBIC, eps=0.0)
    np.testing.assert_allclose(got_t, want.T, atol=1e-13)


def test_quintic_is_not_the_polar_factor_but_keeps_its_directions():
    # The quintic only pushes singular values into a band: its output shares
    # the polar factor's singular vectors, and U^T O V is diagonal.
    m, want = read_fixture("polar_wide_2x3.txt")
    got = oracle.newton_schulz(m, 5, oracle.QUINTIC, eps=0.0)
    u, s, vt = np.linalg.svd(m, full_matrices=False)
    core = u.T @ got @ vt.T
    assert abs(core[0, 1]) < 1e-12 and abs(core[1, 0]) < 1e-12
    assert np.all((np.diag(core) > 0.6) & (np.diag(core) < 1.25))
    assert np.abs(got - want).max() > 1e-3  # 5 quintic steps are a band, not convergence
