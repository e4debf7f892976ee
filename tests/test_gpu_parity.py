"""Parity of the HIP path with the CPU oracle, through the C ABI, on the GPU.

Sizes here finish in seconds on the oracle and still span several 256x256
tiles with ragged tails, both orientations (wide and tall), square matrices,
single rows and columns.  Full-size workloads are in test_gpu_fullsize.py.
"""
import math

import numpy as np
import pytest
import torch

import newton_schulz_03_amd as nsa
import oracle
import workloads
from parity_util import (TOL, check_blocks, device_inputs, host_f64, momentum_within_rounding,
                         rel_fro, singular_values, update_step)
from rounding_bounds import ns_with_bound

pytestmark = pytest.mark.gpu

RAGGED = [(300, 700), (700, 300), (257, 771), (512, 512), (520, 1040), (1040, 520), (33, 65),
          (1, 300), (300, 1), (1, 1), (97, 97), (256, 768)]


def _wl(kind, dtype, shapes, **kw):
    base = workloads.Workload(name="t", dtype=dtype, shapes=tuple(shapes),
                              call="ns" if kind == "gauss" else "step", kind=kind, seed=77)
    import dataclasses
    return dataclasses.replace(base, **kw)


def _ns_check(dtype, shapes, steps=5, coeffs=oracle.QUINTIC, tol=None, eps=1e-7, cu_budget=0):
    """Orthogonalize a Gaussian batch and hold every 256 x 256 block of every
    output to the tolerance against the oracle."""
    wl = _wl("gauss", dtype, shapes, steps=steps, coeffs=coeffs)
    ins = device_inputs(wl)
    xs = [d["x"] for d in ins]
    outs = nsa.ns_batched(xs, steps=steps, coeffs=coeffs, eps=eps, cu_budget=cu_budget)
    torch.cuda.synchronize()
    tol = TOL[dtype] if tol is None else tol
    errs = []
    for x, o, sh in zip(xs, outs, shapes):
        want = oracle.newton_schulz(host_f64(x), steps, coeffs, eps)
        errs.append(check_blocks(host_f64(o), want, tol, what=f"{dtype} {sh}"))
    return errs


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()


def test_c1_fp32_quintic_and_band():
    wl = workloads.standard_workloads()["c1_fp32_256x512"]
    x = device_inputs(wl)[0]["x"]
    o = nsa.ns_batched([x], steps=5)[0]
    want = oracle.newton_schulz(host_f64(x), 5)
    assert rel_fro(host_f64(o), want) <= TOL["fp32"]
    sv = singular_values(host_f64(o))
    assert 0.6818 <= sv.min() and sv.max() <= 1.1344


def test_c1_fp32_cubic30_polar():
    import scipy.linalg

    wl = workloads.c1_cubic()
    x = device_inputs(wl)[0]["x"]
    o = nsa.ns_batched([x], steps=30, coeffs=oracle.CUBIC)[0]
    xh = host_f64(x)
    assert rel_fro(host_f64(o), oracle.newton_schulz(xh, 30, oracle.CUBIC)) <= TOL["fp32"]
    assert rel_fro(host_f64(o), scipy.linalg.polar(xh)[0]) <= TOL["fp32"]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_ns_ragged_batch(dtype):
    _ns_check(dtype, RAGGED)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_ns_one_large_among_many_small(dtype):
    """Tiles of very unequal cost in one launch: the XCD ranges, cut by work,
    hold one-tile matrices on either side of a 48-tile one, and the grid has
    about twice as many workgroups as tiles (the surplus exits at once, or
    after finding every pool of run-time tiles empty)."""
    shapes = [(64, 96)] * 20 + [(1536, 2048)] + [(96, 64)] * 20 + [(1024, 300)]
    _ns_check(dtype, shapes)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("shapes", [
    [(1100, 2304)] * 6,                      # every phase uniform: tiles find their matrix by division
    [(2304, 1100)] * 3 + [(1100, 2304)] * 3,  # the matrix-core phases uniform, the prepare blocks not
    [(1100, 2304)] * 5 + [(1100, 1800)],      # one long side off: every phase ragged again
])
def test_ns_uniform_and_mixed_phases(dtype, shapes):
    """A batch of equal matrices takes a per-matrix block count instead of the
    prefix-table lookup; tall and wide matrices of the same sides share the
    matrix-core phases' counts but not the momentum pass's.  Multi-tile
    matrices with ragged edges, checked per block against the oracle."""
    _ns_check(dtype, shapes)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("eps", [0.0, 1.0])
@pytest.mark.parametrize("steps", [0, 5])
def test_eps_enters_the_normalization(dtype, eps, steps):
    """X0 = U / (||U||_F + eps) with ||U||_F = 0.8: eps = 1 shrinks X0 to 0.44 of
    the unit-norm iterate, so a normalization that dropped eps, or a first Gram
    or product that took the wrong power of the factor, lands far from the
    oracle.  With no iterations the output is X0 itself."""
    rng = np.random.default_rng(31)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    xs = []
    for r, c in [(300, 700), (700, 300), (256, 256)]:
        x = rng.standard_normal((r, c))
        xs.append(torch.from_numpy((0.8 * x / np.linalg.norm(x)).astype(np.float32)).to(tdt).cuda())
    outs = nsa.ns_batched(xs, steps=steps, eps=eps)
    torch.cuda.synchronize()
    for x, o in zip(xs, outs):
        want = oracle.newton_schulz(host_f64(x), steps, oracle.QUINTIC, eps)
        assert rel_fro(host_f64(o), want) <= TOL[dtype], (x.shape, rel_fro(host_f64(o), want))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_many_small_matrices(dtype):
    """A batch of 3000 matrices of up to 40 x 40: past the size at which blocks
    find their matrix by binary search instead of a block-wide scan, with one
    tile per matrix in every phase.

    fp32 runs the quintic for 5 steps against the oracle at 1e-4.  In bf16 the
    5-step quintic is not held to 2e-2 on matrices this small: with only a few
    singular directions, one that sits where the iterated polynomial is steep
    decides the error (5e-2 measured on well-conditioned 40 x 40 inputs).  bf16
    therefore checks maps whose error is bounded by their roundings alone,
    through the same kernels: no iteration (X0: one rounding, 2^-9 relative),
    and one step of (a, b, c) = (0, 1, 0) (X0 X0^T X0: the Gram and the fused
    first-and-last product) and of (0, 0, 1) (A^2 X0: with A^2 too), a few
    roundings each with no cancellation.
    """
    rng = np.random.default_rng(2024)
    xs, hosts = [], []
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for _ in range(3000):
        r, c = (int(v) for v in rng.integers(1, 41, size=2))
        t = torch.from_numpy(rng.standard_normal((r, c)).astype(np.float32)).to(tdt)
        xs.append(t.cuda())
        hosts.append(host_f64(t))
    runs = ([(5, oracle.QUINTIC, TOL["fp32"])] if dtype == "fp32" else
            [(0, oracle.QUINTIC, 2.0 ** -8), (1, (0.0, 1.0, 0.0), TOL["bf16"]),
             (1, (0.0, 0.0, 1.0), TOL["bf16"])])
    for steps, coeffs, tol in runs:
        outs = nsa.ns_batched(xs, steps=steps, coeffs=coeffs)
        torch.cuda.synchronize()
        errs = [rel_fro(host_f64(o), oracle.newton_schulz(h, steps, coeffs))
                for o, h in zip(outs, hosts)]
        assert max(errs) <= tol, (steps, coeffs, max(errs))


@pytest.mark.parametrize("dtype,steps,call", [("bf16", 5, "step"), ("bf16", 1, "ns"),
                                             ("fp32", 5, "step"), ("bf16", 0, "step"),
                                             ("fp32", 0, "ns")])
def test_launch_sequence(dtype, steps, call):
    """Which kernels one call launches: the first product takes the norm factor
    (its iterate is U), bf16 fuses the update into the last product, fp32 and
    zero iterations end with the finish pass."""
    wl = _wl("muon" if call == "step" else "gauss", dtype, [(300, 700), (700, 300)], steps=steps)
    ins = device_inputs(wl)
    torch.cuda.synchronize()
    nsa.timing_reset()
    nsa.timing_enable(True)
    try:
        if call == "step":
            nsa.step_batched([d["w"] for d in ins], [d["g"] for d in ins], [d["m"] for d in ins],
                             steps=steps)
        else:
            nsa.ns_batched([d["x"] for d in ins], steps=steps)
        torch.cuda.synchronize()
    finally:
        nsa.timing_enable(False)
    got = {k: n for k, (_, n) in nsa.timing_read().items() if n}
    fused = dtype == "bf16" and steps > 0
    want = {"prepare": 1, "norm": 1}
    if steps:
        want.update(gram=steps, poly=steps)
        want["prod_finish" if fused and steps == 1 else "prod_first"] = 1
        middle = steps - 1 - (1 if fused and steps > 1 else 0)
        if middle:
            want["prod"] = middle
        if fused and steps > 1:
            want["prod_finish"] = 1
    if not fused:
        want["finish"] = 1
    assert got == want


# Batches for the elementwise bound test.  WIDE_TILES: every padded long side is
# a multiple of 384, so the first and middle products of a bf16 call run in
# 256 x 384 tiles; SQUARE_TILES: not, so every product runs in 256 x 256 tiles.
# Both span several tiles with ragged tails, in both orientations.
WIDE_TILES = [(300, 700), (700, 300), (1000, 1500), (1500, 1000), (40, 1300), (600, 740)]
SQUARE_TILES = [(520, 1040), (1040, 520), (257, 771), (33, 65), (600, 600), (1, 300)]
# Iterations whose terms do not cancel, so that the first-order rounding bound
# is tight enough to gate every element: one to three steps with a positive
# polynomial (Gram, A^2 with its (b/c) A term, the a X term), the a X term
# alone over two steps, and one step of the Gram and product alone.
BOUND_CASES = [((0.5, 0.25, 0.125), 1), ((0.5, 0.25, 0.125), 2), ((0.5, 0.25, 0.125), 3),
               ((1.0, 0.0, 0.0), 2), ((0.0, 1.0, 0.0), 1)]


def _check_bound(got, u, steps, coeffs, what, extra_rel=0.0):
    """Every element of got (float64) within the rounding bound of the exact
    iteration on the bf16 input u, which must be the oracle's result."""
    want = oracle.newton_schulz(u, steps, coeffs)
    x, e = ns_with_bound(u, steps, coeffs)
    assert np.max(np.abs(x - want)) <= 1e-12 * max(1.0, np.max(np.abs(want))), what
    bound = e + extra_rel * (np.abs(want) + e)
    ratio = np.abs(got - want) / np.where(bound > 0, bound, np.inf)
    bad = np.abs(got - want) > bound
    assert not bad.any(), (what, int(bad.sum()), float(np.max(ratio)),
                           tuple(int(i) for i in np.argwhere(bad)[0]))
    return float(np.max(ratio))


@pytest.mark.parametrize("budget", [0, 24])
@pytest.mark.parametrize("batch", ["wide_tiles", "square_tiles"])
@pytest.mark.parametrize("coeffs,steps", BOUND_CASES)
def test_bf16_every_element_within_rounding_bound(coeffs, steps, batch, budget):
    """bf16 products checked element by element: the output of the
    orthogonalize-only call, and the step's own O (read back from a step with
    W = 0, M = 0, where W' = rnd(-lr*scale*O)), each within the first-order
    rounding bound around the oracle's result.  Covers the first, middle and
    fused last products in both tile widths, the Gram's mirror stores and
    diagonal tiles, A^2 with its (b/c) A term, both orientations, and with a CU
    budget the looping kernels."""
    shapes = WIDE_TILES if batch == "wide_tiles" else SQUARE_TILES
    wl = _wl("gauss", "bf16", shapes, steps=steps, coeffs=coeffs)
    xs = [d["x"] for d in device_inputs(wl)]
    outs = nsa.ns_batched(xs, steps=steps, coeffs=coeffs, cu_budget=budget)
    wz = [torch.zeros_like(x) for x in xs]
    mz = [torch.zeros_like(x) for x in xs]
    lr = 0.5
    nsa.step_batched(wz, xs, mz, lr=lr, beta=0.95, steps=steps, coeffs=coeffs, cu_budget=budget)
    torch.cuda.synchronize()
    worst = 0.0
    for x, o, w1, m1, sh in zip(xs, outs, wz, mz, shapes):
        u = host_f64(x)
        assert torch.equal(m1, x), sh  # M' = 0.95 * 0 + G exactly
        worst = max(worst, _check_bound(host_f64(o), u, steps, coeffs, ("ns", sh)))
        # W' = rnd(0 - step * O_stored) with step = lr * scale formed in fp32: one more
        # bf16 rounding and a few fp32 ones on top of O's own bound
        o_step = -host_f64(w1) / update_step(*sh, lr)
        worst = max(worst, _check_bound(o_step, u, steps, coeffs, ("step", sh),
                                        extra_rel=2.0 ** -8 + 4 * 2.0 ** -24))
    print(f"  worst |error| / bound = {worst:.3f}")


@pytest.mark.parametrize("coeffs,steps", [((1.0, 0.0, 0.0), 1), ((0.0, 1.0, 0.0), 1),
                                          ((0.0, 0.0, 1.0), 1), ((0.5, 0.25, -0.125), 2),
                                          (oracle.QUINTIC, 0)])
def test_ns_pieces_fp32(coeffs, steps):
    """Gram, polynomial and product in isolation: X, A X, A^2 X, and steps = 0 (X0)."""
    _ns_check("fp32", [(300, 700), (700, 300), (512, 512)], steps=steps, coeffs=coeffs, tol=1e-5)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_ns_cubic_skips_square(dtype):
    _ns_check(dtype, [(300, 700), (700, 300)], steps=8, coeffs=oracle.CUBIC)


@pytest.mark.parametrize("dtype,nesterov", [("bf16", False), ("bf16", True), ("fp32", False),
                                            ("fp32", True)])
@pytest.mark.parametrize("steps", [5, 1])
def test_step_parity(dtype, nesterov, steps):
    """Full steps against the oracle.  steps = 1: in bf16 the one product is both
    the first (it takes the norm factor) and the last (it writes W)."""
    shapes = [(300, 700), (700, 300), (256, 768), (513, 257)]
    wl = _wl("muon", dtype, shapes, nesterov=nesterov)
    ins = device_inputs(wl)
    w = [d["w"] for d in ins]
    g = [d["g"] for d in ins]
    m = [d["m"] for d in ins]
    w0 = [host_f64(t) for t in w]
    g0 = [host_f64(t) for t in g]
    m0 = [host_f64(t) for t in m]
    nsa.step_batched(w, g, m, lr=wl.lr, beta=wl.beta, nesterov=nesterov, steps=steps)
    torch.cuda.synchronize()
    # orthogonalized update of the GPU's own U, through the orthogonalize-only entry point
    us = [(gi.float() + wl.beta * mi.float()).to(gi.dtype) if nesterov else mi.clone()
          for gi, mi in zip(g, m)]
    o_gpu = nsa.ns_batched(us, steps=steps)
    torch.cuda.synchronize()
    for i, (r, c) in enumerate(shapes):
        w_ref, m_ref, o_ref = oracle.muon_step(w0[i], g0[i], m0[i], lr=wl.lr, beta=wl.beta,
                                               nesterov=nesterov, steps=steps)
        assert rel_fro(host_f64(m[i]), m_ref) <= TOL[dtype] / 4
        check_blocks(host_f64(o_gpu[i]), o_ref, TOL[dtype], what=f"{dtype} step O {(r, c)}")
        # W' is the stored rounding of W - lr*scale*O evaluated in fp32: within one ulp of
        # the result, plus fp32 evaluation error relative to the operands (lr and the
        # product are rounded to fp32, which matters where W and lr*scale*O cancel)
        scale = math.sqrt(max(1.0, r / c))
        upd = wl.lr * scale * host_f64(o_gpu[i])
        expect = w0[i] - upd
        got = host_f64(w[i])
        ulp = np.spacing(np.maximum(np.abs(expect), np.abs(got)).astype(np.float32)).astype(np.float64)
        if dtype == "bf16":
            ulp = ulp * 2.0 ** 16
        bound = ulp + 4.0 * 2.0 ** -24 * (np.abs(w0[i]) + np.abs(upd))
        if nesterov:
            # the step forms U = G + beta*M' in fp32, the reference above from U rounded to
            # the dtype: allow for that difference in O (a few times its expected size)
            rms_o = float(np.sqrt(np.mean(host_f64(o_gpu[i]) ** 2)))
            bound = bound + wl.lr * scale * 8.0 * TOL[dtype] * rms_o
        assert np.all(np.abs(got - expect) <= bound), (r, c, float(np.max(np.abs(got - expect) / bound)))
        # the update itself against the oracle's lr*scale*O; in bf16 the stored W'
        # quantizes an update of about two ulps of W, hence the loose bf16 bound
        assert rel_fro(w0[i] - got, w0[i] - w_ref) <= (TOL[dtype] if dtype == "fp32" else 0.3)


def test_determinism_bitwise():
    wl = _wl("muon", "bf16", [(300, 700), (700, 300), (512, 512)])
    ins = device_inputs(wl)
    runs = []
    for _ in range(2):
        w = [d["w"].clone() for d in ins]
        m = [d["m"].clone() for d in ins]
        nsa.step_batched(w, [d["g"] for d in ins], m)
        torch.cuda.synchronize()
        runs.append([t.view(torch.int16).cpu() for t in w + m])
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_resume_from_saved_momentum():
    """Two steps equal one step, a save/restore of (W, M), and a second step."""
    wl = _wl("muon", "bf16", [(300, 700), (700, 300)])
    ins = device_inputs(wl)
    g = [d["g"] for d in ins]
    w1 = [d["w"].clone() for d in ins]
    m1 = [d["m"].clone() for d in ins]
    nsa.step_batched(w1, g, m1)
    nsa.step_batched(w1, g, m1)
    w2 = [d["w"].clone() for d in ins]
    m2 = [d["m"].clone() for d in ins]
    nsa.step_batched(w2, g, m2)
    saved = [t.cpu() for t in w2 + m2]
    w3 = [t.to("cuda") for t in saved[:2]]
    m3 = [t.to("cuda") for t in saved[2:]]
    nsa.step_batched(w3, g, m3)
    torch.cuda.synchronize()
    for a, b in zip(w1 + m1, w3 + m3):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_zero_and_inplace_and_nan():
    torch.manual_seed(1234)
    x = torch.zeros(300, 700, dtype=torch.bfloat16, device="cuda")
    y = torch.randn(260, 300, device="cuda").to(torch.bfloat16)
    z = torch.randn(64, 128, device="cuda").to(torch.bfloat16)
    z[3, 5] = float("nan")
    y_host = host_f64(y)
    outs = nsa.ns_batched([x, y, z], out=[x, y, z.clone()])  # x and y in place
    torch.cuda.synchronize()
    assert torch.count_nonzero(outs[0]) == 0
    assert rel_fro(host_f64(outs[1]), oracle.newton_schulz(y_host, 5)) <= TOL["bf16"]
    assert torch.isnan(outs[2]).all()
    # zero gradient and momentum: zero update
    w = torch.randn(300, 700, device="cuda").to(torch.bfloat16)
    w0 = w.clone()
    g = torch.zeros_like(w)
    m = torch.zeros_like(w)
    nsa.step_batched([w], [g], [m])
    torch.cuda.synchronize()
    assert torch.equal(w.view(torch.int16), w0.view(torch.int16))


def test_validation_enqueues_nothing():
    x = torch.randn(300, 700, device="cuda").to(torch.bfloat16)
    out = torch.full_like(x, 7.0)
    ws = nsa.allocate_workspace([(300, 700)], torch.bfloat16, "cuda")
    small = ws[: ws.numel() // 2]
    with pytest.raises(nsa.MuonError) as e:
        nsa.ns_batched([x], out=[out], workspace=small)
    assert e.value.status == nsa.MUON_ERR_WORKSPACE
    with pytest.raises(nsa.MuonError) as e:
        nsa.ns_batched([x], out=[out], steps=-1, workspace=ws)
    assert e.value.status == nsa.MUON_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_workspace_reuse_across_shapes():
    """A workspace sized for a large batch serves a smaller one; results match fresh runs."""
    big = [(700, 300), (520, 1040)]
    ws = nsa.allocate_workspace(big, torch.bfloat16, "cuda")
    wl = _wl("gauss", "bf16", big)
    xs = [d["x"] for d in device_inputs(wl)]
    a = nsa.ns_batched(xs, workspace=ws)
    b = nsa.ns_batched(xs[:1], workspace=ws)
    c = nsa.ns_batched(xs[:1])
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(b[0].view(torch.int16), c[0].view(torch.int16))


@pytest.mark.parametrize("dtype,nesterov", [("bf16", False), ("bf16", True), ("fp32", False)])
def test_step_momentum_in_host_memory(dtype, nesterov):
    """The momentum kept in pinned host memory gives bit-identical results to
    the momentum in HBM, and both are held to the oracle: M' element by element
    (within its storage rounding), and the step's own O (from a second step
    with W = 0 and the momentum in host memory, which stores rnd(-lr*scale*O))
    per 256 x 256 block."""
    shapes = [(300, 700), (700, 300), (513, 257), (64, 2048)]
    wl = _wl("muon", dtype, shapes, nesterov=nesterov)
    ins = device_inputs(wl)
    w_dev = [d["w"].clone() for d in ins]
    m_dev = [d["m"].clone() for d in ins]
    g = [d["g"] for d in ins]
    w_host = [d["w"].clone() for d in ins]
    m_host = [d["m"].cpu().pin_memory() for d in ins]
    wz = [torch.zeros_like(d["w"]) for d in ins]
    mz_host = [d["m"].cpu().pin_memory() for d in ins]
    nsa.step_batched(w_dev, g, m_dev, lr=wl.lr, beta=wl.beta, nesterov=nesterov, steps=5)
    nsa.step_batched(w_host, g, m_host, lr=wl.lr, beta=wl.beta, nesterov=nesterov, steps=5,
                     momentum_host=True)
    nsa.step_batched(wz, g, mz_host, lr=wl.lr, beta=wl.beta, nesterov=nesterov, steps=5,
                     momentum_host=True)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(w_dev[i], w_host[i]), i
        assert torch.equal(m_dev[i].cpu(), m_host[i]), i
        assert torch.equal(mz_host[i], m_host[i]), i
    for i, sh in enumerate(shapes):
        gh, mh = host_f64(g[i]), host_f64(ins[i]["m"])
        assert not momentum_within_rounding(mh, gh, host_f64(m_host[i]), wl.beta, dtype).any(), sh
        _, _, o_ref = oracle.muon_step(np.zeros_like(gh), gh, mh, lr=wl.lr, beta=wl.beta,
                                       nesterov=nesterov, steps=5)
        o_step = -host_f64(wz[i]) / update_step(*sh, wl.lr)
        # the step rounds M' (and U = G + beta*M' with Nesterov) to the dtype, the
        # oracle keeps them in float64: a difference far below the tolerance
        check_blocks(o_step, o_ref, TOL[dtype], what=f"{dtype} host momentum, step O, {sh}")
    # a second step from the state left in host memory
    nsa.step_batched(w_dev, g, m_dev, lr=wl.lr, beta=wl.beta, nesterov=nesterov, steps=5)
    nsa.step_batched(w_host, g, m_host, lr=wl.lr, beta=wl.beta, nesterov=nesterov, steps=5,
                     momentum_host=True)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(w_dev[i], w_host[i]) and torch.equal(m_dev[i].cpu(), m_host[i]), i


@pytest.mark.parametrize("fp8_steps", [0, 2])
def test_momentum_host_many_chunks(fp8_steps):
    """Enough matrices for many chunks, so that both staging slots are reused
    several times and the copies of neighbouring chunks overlap: bit-identical
    to the momentum in HBM, over two steps (the second call waits for the
    first)."""
    rng = np.random.default_rng(17)
    shapes = [tuple(int(v) for v in rng.choice([256, 513, 768, 1024], size=2)) for _ in range(26)]
    wl = _wl("muon", "bf16", shapes)
    ins = device_inputs(wl)
    g = [d["g"] for d in ins]
    w_dev = [d["w"].clone() for d in ins]
    m_dev = [d["m"].clone() for d in ins]
    w_host = [d["w"].clone() for d in ins]
    m_host = [d["m"].cpu().pin_memory() for d in ins]
    for _ in range(2):
        nsa.step_batched(w_dev, g, m_dev, steps=5, fp8_steps=fp8_steps)
        nsa.step_batched(w_host, g, m_host, steps=5, fp8_steps=fp8_steps, momentum_host=True)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(w_dev[i], w_host[i]), (i, shapes[i])
        assert torch.equal(m_dev[i].cpu(), m_host[i]), (i, shapes[i])


def test_momentum_host_rejects_device_memory():
    wl = _wl("muon", "bf16", [(64, 96)])
    d = device_inputs(wl)[0]
    lib = nsa.load_library()
    from newton_schulz_03_amd._binding import NsParams, StepParams, _i64_array, _ptr_array
    import ctypes
    ws = nsa.allocate_workspace([(64, 96)], torch.bfloat16, "cuda", momentum_host=True)
    p = StepParams(0.02, 0.95, 0, NsParams(5, 3.4445, -4.775, 2.0315, 1e-7), 1)
    st = lib.muon_step_batched(1, _i64_array([64]), _i64_array([96]), _ptr_array([d["w"].data_ptr()]),
                               _ptr_array([d["g"].data_ptr()]), _ptr_array([d["m"].data_ptr()]), 0,
                               ctypes.byref(p), ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert st == nsa.MUON_ERR_INVALID_ARG and "pinned host" in nsa.last_error_detail()


def test_ns_on_second_stream_during_gemm_load_is_unchanged():
    """The orthogonalization on its own stream, while bf16 products run on another
    (default priorities), gives the same bits as alone."""
    wl = _wl("gauss", "bf16", [(512, 1536), (1536, 512), (1024, 1024)])
    xs = [d["x"] for d in device_inputs(wl)]
    alone = nsa.ns_batched(xs, steps=5)
    torch.cuda.synchronize()
    a = torch.randn(4096, 6144, device="cuda").to(torch.bfloat16)
    b = (torch.randn(6144, 2048, device="cuda") * 0.02).to(torch.bfloat16)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(sa):
        for _ in range(20):
            torch.matmul(a, b)
    with torch.cuda.stream(sb):
        both = nsa.ns_batched(xs, steps=5)
    torch.cuda.synchronize()
    for x, y in zip(alone, both):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_maximum_dimension(dtype):
    """The longest side the ABI accepts (65536), both orientations, against the oracle."""
    n = nsa.MAX_DIM
    _ns_check(dtype, [(3, n), (n, 5)])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rank_deficient_inputs(dtype):
    """Rank-1 and rank-deficient matrices.

    Exact zero rows and columns stay exactly zero.  Directions of the null
    space are not fixed by the input: rounding (the input's to the dtype, and
    each product's) puts noise there that each step multiplies by up to
    a = 3.4445, so several outputs are correct in them.  The oracle check is
    therefore on the input directions with normalized singular value >= 1e-2
    (to 2e-2 in bf16, 1e-4 in fp32).  In fp32 the whole output is also bounded:
    1e-7 rounding times a^4 over a few hundred null directions is a few 1e-4,
    so the full-matrix error must stay below 1e-3.
    """
    rng = np.random.default_rng(5)
    mats = []
    u = rng.standard_normal((300, 1)); v = rng.standard_normal((1, 700))
    mats.append(u @ v)                                # rank 1, wide
    b = rng.standard_normal((520, 40)) @ rng.standard_normal((40, 260))
    mats.append(b)                                    # rank 40, tall
    z = rng.standard_normal((257, 513)); z[100:, :] = 0.0
    mats.append(z)                                    # zero rows
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    xs = [torch.from_numpy(m.astype(np.float32)).to(tdt).cuda() for m in mats]
    outs = nsa.ns_batched(xs, steps=5)
    torch.cuda.synchronize()
    for x, o in zip(xs, outs):
        xh, oh = host_f64(x), host_f64(o)
        want = oracle.newton_schulz(xh, 5)
        u, sv, vt = np.linalg.svd(xh, full_matrices=False)
        keep = sv / np.linalg.norm(sv) >= 1e-2
        uk, vk = u[:, keep], vt[keep].T
        ref = uk.T @ want @ vk
        assert np.linalg.norm(uk.T @ oh @ vk - ref) / np.linalg.norm(ref) <= TOL[dtype]
        if dtype == "fp32":
            assert rel_fro(oh, want) <= 1e-3
        # rows (columns) of the input that are zero stay exactly zero in the output
        zr = np.all(xh == 0, axis=1)
        zc = np.all(xh == 0, axis=0)
        assert np.all(oh[zr, :] == 0) and np.all(oh[:, zc] == 0)


@pytest.mark.parametrize("case", ["many", "cubic", "long"])
def test_wide_product_tiles_match_square_tiles(case):
    """The first and middle products run in 256 x 384 tiles when every padded
    long side is a multiple of 384; a CU budget (here larger than any grid)
    selects the 256 x 256 kernel instead.  Both accumulate every element with
    the same MFMAs in the same order, so the outputs agree bit for bit.
    many: 2100 matrices, past the batch size at which blocks find their matrix
    by binary search; cubic: (1.5, -0.5, 0), where the product reads A itself;
    long: a long side of 65280 = 170 x 384, near the largest allowed, in both
    orientations."""
    rng = np.random.default_rng(99)
    if case == "many":
        shapes = []
        for _ in range(2100):
            s, l = int(rng.integers(1, 41)), int(rng.integers(513, 769))
            shapes.append((s, l) if rng.integers(2) else (l, s))
        coeffs = oracle.QUINTIC
    elif case == "cubic":
        shapes = [(300, 700), (700, 300), (1000, 1500), (1500, 1000), (256, 768), (33, 700)]
        coeffs = oracle.CUBIC
    else:
        shapes = [(256, 65280), (65280, 256)]
        coeffs = oracle.QUINTIC
    xs = [torch.from_numpy(rng.standard_normal(sh).astype(np.float32)).to(torch.bfloat16).cuda()
          for sh in shapes]
    wide = nsa.ns_batched(xs, steps=5, coeffs=coeffs)
    square = nsa.ns_batched(xs, steps=5, coeffs=coeffs, cu_budget=1 << 20)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(wide, square)):
        assert torch.equal(a, b), (i, shapes[i])
    # the larger ones against the oracle too (the small ones' bf16 error is
    # discussed at test_many_small_matrices)
    for i, sh in enumerate(shapes):
        if min(sh) >= 256:
            want = oracle.newton_schulz(host_f64(xs[i]), 5, coeffs)
            assert rel_fro(host_f64(wide[i]), want) <= TOL["bf16"], (i, sh)


@pytest.mark.parametrize("steps", [2, 3])
def test_wide_first_product_feeds_square_last_product(steps):
    """With 2 steps the wide first product hands its iterate straight to the
    256 x 256 fused last product; with 3 one wide middle product sits between.
    Orthogonalization and full step, bit for bit against the 256 x 256 path."""
    shapes = [(300, 700), (700, 300), (1024, 1536), (513, 257)]
    wl = _wl("muon", "bf16", shapes)
    ins = device_inputs(wl)
    g = [d["g"] for d in ins]
    wide = nsa.ns_batched(g, steps=steps)
    square = nsa.ns_batched(g, steps=steps, cu_budget=1 << 20)
    w0 = [d["w"].clone() for d in ins]
    m0 = [d["m"].clone() for d in ins]
    w1 = [d["w"].clone() for d in ins]
    m1 = [d["m"].clone() for d in ins]
    nsa.step_batched(w0, g, m0, steps=steps, nesterov=True)
    nsa.step_batched(w1, g, m1, steps=steps, nesterov=True, cu_budget=1 << 20)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(wide[i], square[i]), i
        assert torch.equal(w0[i], w1[i]) and torch.equal(m0[i], m1[i]), i
    for i, sh in enumerate(shapes):
        want = oracle.newton_schulz(host_f64(g[i]), steps)
        assert rel_fro(host_f64(wide[i]), want) <= TOL["bf16"], (i, sh)


@pytest.mark.parametrize("budget", [8, 24, 100])
def test_cu_budget_gives_identical_results(budget):
    """A CU budget (fewer workgroups, each looping over tiles) changes only where
    tiles run: the bits are the same, for the orthogonalization and the step.
    The looping kernels' results are also held to the oracle directly: every
    256 x 256 block of the orthogonalization, of the step's own O (a step with
    W = 0 stores rnd(-lr*scale*O)) and the momentum element by element."""
    shapes = [(300, 700), (700, 300), (1024, 1536), (513, 257)]
    wl = _wl("muon", "bf16", shapes)
    ins = device_inputs(wl)
    g = [d["g"] for d in ins]
    full = nsa.ns_batched(g, steps=5)
    some = nsa.ns_batched(g, steps=5, cu_budget=budget)
    w0 = [d["w"].clone() for d in ins]
    m0 = [d["m"].clone() for d in ins]
    w1 = [d["w"].clone() for d in ins]
    m1 = [d["m"].clone() for d in ins]
    nsa.step_batched(w0, g, m0, steps=5)
    nsa.step_batched(w1, g, m1, steps=5, cu_budget=budget)
    wz = [torch.zeros_like(t) for t in w1]
    mz = [d["m"].clone() for d in ins]
    nsa.step_batched(wz, g, mz, steps=5, cu_budget=budget, lr=wl.lr)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(full[i], some[i]), i
        assert torch.equal(w0[i], w1[i]) and torch.equal(m0[i], m1[i]), i
        assert torch.equal(mz[i], m1[i]), i
    for i, sh in enumerate(shapes):
        gh, mh = host_f64(g[i]), host_f64(ins[i]["m"])
        check_blocks(host_f64(some[i]), oracle.newton_schulz(gh, 5), TOL["bf16"],
                     what=f"ns, budget {budget}, {sh}")
        assert not momentum_within_rounding(mh, gh, host_f64(m1[i]), wl.beta, "bf16").any(), sh
        _, _, o_ref = oracle.muon_step(np.zeros_like(gh), gh, mh, lr=wl.lr, beta=wl.beta, steps=5)
        o_step = -host_f64(wz[i]) / update_step(*sh, wl.lr)
        check_blocks(o_step, o_ref, TOL["bf16"], what=f"step O, budget {budget}, {sh}")


def _up(x, a):
    return -(-x // a) * a


def _workspace_sym(ws, shape):
    """A = X X^T and B = c A^2 + b A of the only matrix of a one-matrix bf16 call,
    read from the workspace (layout in muon_abi.hip: descriptor table, the 7
    phase prefix arrays, the inverse norm, two sets of 16 tile-claim counters,
    the momentum-pass partials, X ping, X pong, A, B; matrices in 256 x 32 slabs)
    as s_pad x s_pad int16 arrays."""
    r, c = shape
    tall = r > c
    sp, lp = _up(min(shape), 256), _up(max(shape), 256)
    blocks = (sp // 256) * (lp // 64) if tall else (sp // 32) * (lp // 256)
    off = _up(112, 256) + _up(4 * 7 * 2, 256) + _up(4, 256) + _up(4 * 2 * 16, 256)
    off += _up(4 * blocks, 256)
    off += 2 * _up(sp * lp * 2, 256)
    raw = ws.view(torch.int16)
    out = []
    for k in range(2):
        n = sp * sp
        slabs = raw[off // 2:off // 2 + n].cpu().numpy().reshape(sp // 256, sp // 32, 256, 32)
        out.append(slabs.transpose(0, 2, 1, 3).reshape(sp, sp))
        off += _up(n * 2, 256)
    return out


@pytest.mark.parametrize("shape", [(300, 700), (1040, 520), (1536, 1600)])
def test_gram_and_square_are_exactly_symmetric(shape):
    """The stored A and B are bitwise symmetric: off-diagonal tiles store their
    mirror, and diagonal tiles form only the blocks on and above the diagonal and
    mirror them.  Also each is within the bf16 tolerance of the oracle's A and
    c A^2 + b A of the first step."""
    x = torch.from_numpy(np.random.default_rng(11).standard_normal(shape).astype(np.float32))
    x = x.to(torch.bfloat16).cuda()
    ws = nsa.allocate_workspace([shape], torch.bfloat16, "cuda")
    nsa.ns_batched([x], steps=1, workspace=ws)
    torch.cuda.synchronize()
    a, b = _workspace_sym(ws, shape)
    assert np.array_equal(a, a.T) and np.array_equal(b, b.T)
    u = host_f64(x)
    u = u.T if shape[0] > shape[1] else u
    x0 = u / (np.linalg.norm(u) + 1e-7)
    s = x0.shape[0]
    _, qb, qc = oracle.QUINTIC
    a_ref = x0 @ x0.T
    b_ref = qc * (a_ref @ a_ref) + qb * a_ref
    bf = lambda v: torch.from_numpy(v.astype(np.int16)).view(torch.bfloat16).double().numpy()
    check_blocks(bf(a)[:s, :s], a_ref, TOL["bf16"], what=f"A {shape}")
    check_blocks(bf(b)[:s, :s], b_ref, TOL["bf16"], what=f"B {shape}")


def test_launch_sequence_momentum_host():
    """A step with the momentum in host memory runs the step's kernels once per
    chunk, and copies each chunk's momentum in and out once (timed on the copy
    streams)."""
    shapes = [(300, 700), (700, 300), (256, 512), (512, 256), (640, 640)]
    wl = _wl("muon", "bf16", shapes)
    ins = device_inputs(wl)
    m_host = [d["m"].cpu().pin_memory() for d in ins]
    ws = nsa.allocate_workspace(shapes, torch.bfloat16, "cuda", momentum_host=True)
    torch.cuda.synchronize()
    nsa.timing_reset()
    nsa.timing_enable(True)
    try:
        nsa.step_batched([d["w"] for d in ins], [d["g"] for d in ins], m_host, steps=2,
                         workspace=ws, momentum_host=True)
        torch.cuda.synchronize()
    finally:
        nsa.timing_enable(False)
    got = {k: n for k, (_, n) in nsa.timing_read().items() if n}
    chunks = got["prepare"]
    assert 1 < chunks <= 16, got
    want = {"prepare": chunks, "norm": chunks, "gram": 2 * chunks, "poly": 2 * chunks,
            "prod_first": chunks, "prod_finish": chunks, "mom_in": chunks, "mom_out": chunks}
    assert got == want
