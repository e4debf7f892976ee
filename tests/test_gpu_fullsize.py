"""Full-size workloads through the C ABI, in the launch configuration of the benchmark.

Each workload runs whole, in one call, at its real size. The float64 oracle
then checks sampled matrices one by one, every 256 x 256 block of them. The
step's own orthogonalized update O is read back from a second step over the
same batch with W = 0 (which stores rnd(-lr*scale*O)), so the O compared with
the oracle is the one the step applied, not one recomputed by another call.
Every matrix of the batch is also checked through properties that hold at any
size:

- momentum on sampled elements of every matrix, against the oracle's formula
  applied to those elements;
- finiteness;
- the energy band of the orthogonalized output.

Progress lines go to the real stderr, because one of these tests can take
about a minute (input generation and the oracle on the host).
"""
import math
import sys
import time

import numpy as np
import pytest
import torch

import newton_schulz_03_amd as nsa
import oracle
import workloads
from parity_util import (TOL, check_blocks, device_inputs, host_f64, momentum_within_rounding,
                         rel_fro, singular_values, update_step)

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]

_T0 = time.time()
_CAPMAN = None


def progress(msg):
    """One line on the real stderr, with pytest's output capture suspended for it."""
    line = f"[fullsize {time.time() - _T0:7.1f}s] {msg}\n"
    if _CAPMAN is not None:
        with _CAPMAN.global_and_fixture_disabled():
            sys.stderr.write(line)
            sys.stderr.flush()
    else:
        sys.stderr.write(line)
        sys.stderr.flush()


@pytest.fixture(autouse=True)
def _announce(request):
    global _CAPMAN
    _CAPMAN = request.config.pluginmanager.getplugin("capturemanager")
    progress(f"start {request.node.name}")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    progress(f"end {request.node.name}")


# Quintic band (oracle pin): after 5 steps every normalized singular value at
# least 5.18e-3 lands in [0.6818, 1.1344]; nothing leaves (0, 1.2024].  A
# Gaussian matrix with unequal sides has all its normalized singular values
# above that threshold (2048x6144: about 9e-3; 6144x1024: about 1.8e-2), so
# ||O||_F^2 / s lies in [0.6818^2, 1.1344^2]; bf16 rounding moves it slightly.
# A square Gaussian matrix has singular values near zero, so only the upper
# bound holds there.
ENERGY_BAND = (0.6818 ** 2 * 0.97, 1.1344 ** 2 * 1.03)


def _energy_per_dim(o):
    s = min(o.shape)
    return float(o.float().pow(2).sum().item()) / s


def _check_energy(o, j):
    e = _energy_per_dim(o)
    lo = ENERGY_BAND[0] if o.shape[0] != o.shape[1] else 0.0
    assert lo <= e <= ENERGY_BAND[1], (j, tuple(o.shape), e)


def _momentum_elements(wl, m0_dev, g_dev, m1_dev, j, count=4096):
    """M' of matrix j at `count` seeded random positions, HIP against the oracle."""
    rows, cols = wl.shapes[j]
    rng = np.random.default_rng([wl.seed, j, 1000])
    idx = torch.from_numpy(rng.integers(0, rows * cols, size=count)).to(g_dev.device)
    pick = lambda t: host_f64(t.reshape(-1)[idx])
    m0, g = pick(m0_dev), pick(g_dev)
    assert np.array_equal(oracle.momentum(m0, g, wl.beta), wl.beta * m0 + g)
    bad = momentum_within_rounding(m0, g, pick(m1_dev), wl.beta, wl.dtype)
    assert not bad.any(), (j, int(bad.sum()))


def _check_step_sample(wl, j, w_dev, m_dev, o_step_dev, o_ns_dev):
    """Oracle step on matrix j's regenerated inputs against the HIP results:
    M' and both O (the step's own, and the orthogonalize-only call's on the
    step's M') per 256 x 256 block, W' within its rounding."""
    raw = workloads.matrix_inputs(wl, j)
    w0, m0, g0 = (host_f64(workloads.cast(raw[k], wl.dtype)) for k in ("w", "m", "g"))
    w_ref, m_ref, o_ref = oracle.muon_step(w0, g0, m0, lr=wl.lr, beta=wl.beta,
                                           nesterov=wl.nesterov, steps=wl.steps,
                                           coeffs=wl.coeffs, eps=wl.eps)
    rows, cols = wl.shapes[j]
    m1 = host_f64(m_dev)
    o_ns = host_f64(o_ns_dev)
    o_step = -host_f64(o_step_dev) / update_step(rows, cols, wl.lr)
    w1 = host_f64(w_dev)
    e_m = rel_fro(m1, m_ref)
    e_step = check_blocks(o_step, o_ref, TOL[wl.dtype], what=f"matrix {j} step O")
    e_ns = check_blocks(o_ns, o_ref, TOL[wl.dtype], what=f"matrix {j} ns O")
    progress(f"  matrix {j} {wl.shapes[j]}: M' err {e_m:.2e}, step O worst block {e_step:.2e} "
             f"(whole {rel_fro(o_step, o_ref):.2e}), ns O worst block {e_ns:.2e}")
    assert e_m <= TOL[wl.dtype] / 4
    # W' is the stored rounding of W - lr*scale*O, O the step's own
    upd = update_step(rows, cols, wl.lr) * o_step
    expect = w0 - upd
    ulp = np.spacing(np.maximum(np.abs(expect), np.abs(w1)).astype(np.float32)).astype(np.float64)
    ulp *= 2.0 ** 16 if wl.dtype == "bf16" else 1.0
    # O read back from W'_zero = rnd(-step*O) carries one more rounding of the update
    bound = 1.5 * ulp + 4.0 * 2.0 ** -24 * (np.abs(w0) + np.abs(upd)) + \
        2.0 ** -8 * np.abs(upd) * (1.0 if wl.dtype == "bf16" else 2.0 ** -16)
    assert np.all(np.abs(w1 - expect) <= bound), (j, float(np.max(np.abs(w1 - expect) / bound)))
    assert rel_fro(w0 - w1, w0 - w_ref) <= 0.3


def _step32(wl, j):
    """lr * sqrt(max(1, rows/cols)) as the kernel forms it: both factors and the
    product in fp32."""
    rows, cols = wl.shapes[j]
    scale = np.float32(math.sqrt(max(1.0, rows / cols)))
    return float(np.float32(np.float32(wl.lr) * scale))


def _run_full_step(wl, samples):
    progress(f"{wl.name}: generating {wl.batch} matrices")
    ins = device_inputs(wl)
    w = [d["w"] for d in ins]
    g = [d["g"] for d in ins]
    m = [d["m"] for d in ins]
    m0 = [t.clone() for t in m]
    progress(f"{wl.name}: step over the whole batch")
    nsa.step_batched(w, g, m, lr=wl.lr, beta=wl.beta, nesterov=wl.nesterov, steps=wl.steps,
                     coeffs=wl.coeffs, eps=wl.eps)
    # the same step with W = 0 (and the same M): W' = rnd(-lr*scale*O) carries the
    # step's own O at the dtype's relative precision
    wz = [torch.zeros_like(t) for t in w]
    mz = [t.clone() for t in m0]
    nsa.step_batched(wz, g, mz, lr=wl.lr, beta=wl.beta, nesterov=wl.nesterov, steps=wl.steps,
                     coeffs=wl.coeffs, eps=wl.eps)
    torch.cuda.synchronize()
    for j in range(wl.batch):
        assert torch.equal(mz[j], m[j]), j
    del mz
    # O of the step's own U (U = M' without Nesterov) through the orthogonalize-only call
    assert not wl.nesterov
    o = nsa.ns_batched(m, steps=wl.steps, coeffs=wl.coeffs, eps=wl.eps)
    torch.cuda.synchronize()
    progress(f"{wl.name}: whole-batch properties")
    for j in range(wl.batch):
        _momentum_elements(wl, m0[j], g[j], m[j], j)
        assert torch.isfinite(w[j]).all() and torch.isfinite(o[j]).all(), j
        _check_energy(o[j], j)
        # the step applied the very O that the orthogonalize-only call computes from
        # M': W'_zero = rnd(-(step * O)), with step = lr * scale formed in fp32
        assert torch.equal(wz[j], (o[j].float() * -_step32(wl, j)).to(wz[j].dtype)), j
    del m0, g
    for j in samples:
        _check_step_sample(wl, j, w[j], m[j], wz[j], o[j])


def test_c2_full_step():
    wl = workloads.standard_workloads()["c2_96x2048x6144"]
    _run_full_step(wl, samples=[0, 47, 95])


def test_c3_full_step_one_rank_share():
    wl = workloads.standard_workloads()["c3_rank_222_experts"]
    # layer 0 gate (6144x2048, tall), layer 37 up (tall), layer 73 down (wide)
    _run_full_step(wl, samples=[0, 112, 221])


def test_c4_full_ns_dense_and_skinny():
    wl = workloads.standard_workloads()["c4_dense_attn"]
    progress(f"{wl.name}: generating {wl.batch} matrices")
    xs = [d["x"] for d in device_inputs(wl)]
    o = nsa.ns_batched(xs, steps=wl.steps, coeffs=wl.coeffs, eps=wl.eps)
    torch.cuda.synchronize()
    for j in range(wl.batch):
        assert torch.isfinite(o[j]).all(), j
        _check_energy(o[j], j)
    for j in [0, 16, 31]:  # square 6144^2, skinny 6144x1024 (tall)
        x = host_f64(xs[j])
        want = oracle.newton_schulz(x, wl.steps, wl.coeffs, wl.eps)
        worst = check_blocks(host_f64(o[j]), want, TOL[wl.dtype], what=f"matrix {j}")
        progress(f"  matrix {j} {wl.shapes[j]}: O err {rel_fro(host_f64(o[j]), want):.2e}, "
                 f"worst 256 x 256 block {worst:.2e}")


def _bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (float64 tensor; 2^-133 at zero)."""
    _, e = torch.frexp(x.abs().clamp_min(2.0 ** -126))
    return torch.ldexp(torch.ones_like(x), (e - 8).to(torch.int32))


# Workload 5 in bf16: directions whose normalized singular value sits near the
# bf16 noise floor are not fixed by the input.  Rounding U to bf16 (and every
# later rounding) perturbs the normalized singular values by about the
# spectral norm of the rounding error, RES_FLOOR = ||rnd(U) - U||_2 / ||U||_F
# (measured per matrix: 0.8e-4 to 1.6e-4 at these shapes).  A direction with
# sigma = RESOLVED_FACTOR * RES_FLOOR then moves by at most 1/12 of itself, and
# the quintic maps it into its band wherever it lands.  Directions at or above
# that cutoff are "resolved": the output on them is gated to the tolerance,
# and their output singular values to the quintic band.  (A bf16 emulation of
# the iteration on these shapes measured 1.1e-2 to 1.4e-2 on the resolved
# directions, about half of all of them, and 1.7e-2 to 2.2e-2 at a cutoff of
# half this one.)  Below the cutoff several outputs are correct.
RESOLVED_FACTOR = 12.0
# p^10 maps every x >= 1.07e-5 into [0.6818, 1.1344] (oracle pin)
QUINTIC10_BAND = (0.6818, 1.1344)


def _rounding_floor(u_exact, u_stored):
    """||u_stored - u_exact||_2 / ||u_exact||_F (the largest singular value of the
    rounding error, by Lanczos)."""
    import scipy.sparse.linalg

    e = u_stored - u_exact
    top = scipy.sparse.linalg.svds(e, k=1, return_singular_vectors=False)[0]
    return float(top) / float(np.linalg.norm(u_exact))


def _resolved(o, o_ref, u, s, v, tau):
    """Relative error and singular values of the output on the input directions
    whose normalized singular value is >= tau, and how many there are."""
    keep = s / np.linalg.norm(s) >= tau
    uk, vk = u[:, keep], v[:, keep]
    ref = uk.T @ o_ref @ vk
    got = uk.T @ o @ vk
    err = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    return err, singular_values(got), int(keep.sum())


def test_c5_full_step_illconditioned_nesterov():
    wl = workloads.standard_workloads()["c5_mixed_illcond"]
    # sampled matrices: the first of each (short side, orientation) with short side
    # <= 2048 (five of them), and the first with a short side of 6144 (square)
    picks = {}
    for j, (r, c) in enumerate(wl.shapes):
        key = (min(r, c), r > c)
        if min(r, c) <= 2048 and key not in picks:
            picks[key] = j
    samples = sorted(picks.values())[:5]
    samples.append(next(j for j, (r, c) in enumerate(wl.shapes) if min(r, c) == 6144))
    progress(f"{wl.name}: generating {wl.batch} ill-conditioned matrices on the device")
    ins, factors = [], {}
    for j in range(wl.batch):
        d, f = workloads.illcond_inputs_device(wl, j, "cuda")
        ins.append(d)
        if j in samples:
            factors[j] = tuple(t.cpu().numpy() for t in f)
        del f
        if j % 32 == 31:
            torch.cuda.synchronize()
            progress(f"  {j + 1} generated")
    w = [d["w"] for d in ins]
    g = [d["g"] for d in ins]
    m = [d["m"] for d in ins]
    w0 = [t.clone() for t in w]
    progress(f"{wl.name}: step over the whole batch ({wl.steps} NS steps, Nesterov)")
    nsa.step_batched(w, g, m, lr=wl.lr, beta=wl.beta, nesterov=True, steps=wl.steps,
                     coeffs=wl.coeffs, eps=wl.eps)
    # The same step with W = 0: then W' = -lr*scale*O rounded once, which carries the
    # step's own O at the dtype's relative precision (with the workload's W, bf16
    # storage of W' quantizes an update of a few ulps).
    wz = [torch.zeros_like(t) for t in w]
    mz = [torch.zeros_like(t) for t in m]
    nsa.step_batched(wz, g, mz, lr=wl.lr, beta=wl.beta, nesterov=True, steps=wl.steps,
                     coeffs=wl.coeffs, eps=wl.eps)
    torch.cuda.synchronize()
    for j in range(wl.batch):
        # M0 = 0, so M' = G exactly and U = (1 + beta) G
        assert torch.equal(m[j], g[j]) and torch.equal(mz[j], g[j]), j
        assert torch.isfinite(w[j]).all() and torch.isfinite(wz[j]).all(), j
        # W' = rnd(W - t) and W'_zero = rnd(-t) for the same t = lr*scale*O
        w1, a, z = w[j].double(), w0[j].double(), wz[j].double()
        bound = _bf16_ulp(w1) + _bf16_ulp(a + z) + 0.5 * _bf16_ulp(z)
        assert bool(((w1 - (a + z)).abs() <= bound).all()), j
    del mz
    # the orthogonalize-only entry point on U rounded to the dtype, whole batch
    us = [(gi.float() * (1.0 + wl.beta)).to(gi.dtype) for gi in g]
    o = nsa.ns_batched(us, steps=wl.steps, coeffs=wl.coeffs, eps=wl.eps)
    torch.cuda.synchronize()
    for j in range(wl.batch):
        assert torch.isfinite(o[j]).all(), j
        # nothing leaves (0, 1.2024] in exact arithmetic; sum of sigma^2 <= 1.25^2 * s
        assert _energy_per_dim(o[j]) <= 1.25 ** 2, j
    for j in samples:
        rows, cols = wl.shapes[j]
        u, s, v = factors[j]
        w_in, g_in = host_f64(w0[j]), host_f64(g[j])
        progress(f"  matrix {j} {wl.shapes[j]}: oracle")
        _, _, o_ref = oracle.muon_step(w_in, g_in, np.zeros_like(g_in), lr=wl.lr,
                                       beta=wl.beta, nesterov=True, steps=wl.steps,
                                       coeffs=wl.coeffs, eps=wl.eps)
        tau = RESOLVED_FACTOR * _rounding_floor((1.0 + wl.beta) * g_in, host_f64(us[j]))
        checks = {"ns": host_f64(o[j]), "step": -host_f64(wz[j]) / update_step(rows, cols, wl.lr)}
        for name, oj in checks.items():
            err, sv_res, kept = _resolved(oj, o_ref, u, s, v, tau)
            sv = singular_values(oj)
            full = rel_fro(oj, o_ref)
            progress(f"  matrix {j} {wl.shapes[j]} {name}: cutoff {tau:.2e}, resolved {kept} of "
                     f"{min(rows, cols)} dirs, err {err:.2e}, their sigma [{sv_res.min():.4f}, "
                     f"{sv_res.max():.4f}]; all sigma [{sv.min():.3f}, {sv.max():.3f}], "
                     f"full-matrix err {full:.2e} (bf16 floor, not gated)")
            assert err <= TOL[wl.dtype], (j, name, err)
            lo, hi = QUINTIC10_BAND
            assert lo - TOL[wl.dtype] <= sv_res.min() and sv_res.max() <= hi + TOL[wl.dtype], \
                (j, name, sv_res.min(), sv_res.max())
            assert sv.max() <= 1.25 * (1 + 2.0 ** -7), (j, name)
            assert int((sv >= 0.6).sum()) >= kept, (j, name)
