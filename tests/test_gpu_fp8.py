"""The e4m3 steps (fp8_steps) on the GPU, through the C ABI.

- Parity: with fp8_steps = 2 of 5 quintic steps, every 256 x 256 block of the
  output is within the bf16 tolerance of the float64 oracle, and the
  whole-matrix error is within 10% of the bf16 path's on the same input (the
  CPU emulation in test_fp8_feasibility.py found the two equal on these
  shapes).  Orthogonalize-only and full step, wide, tall, ragged, and the
  cubic iteration (no A^2, the product reads A).
- The quantizer, white box: after a call with one e4m3 step, the workspace's
  e4m3 copy of X^T equals the CPU quantization of the input (one power-of-two
  scale per 32 values, the smallest that keeps the block maximum at or below
  448, values rounded to nearest even), byte for byte.
- The whole e4m3 step against a CPU emulation of it (same quantization and
  bf16 rounding points, products in float64): every block within 2e-3.
- Determinism: two calls give the same bits.
"""
import numpy as np
import pytest
import torch

import newton_schulz_03_amd as nsa
import oracle
from parity_util import TOL, block_errors, check_blocks, device_inputs, host_f64, rel_fro
from test_fp8_feasibility import mx_e4m3

pytestmark = pytest.mark.gpu

SHAPES = [(2048, 6144), (6144, 2048), (1024, 3072), (512, 1536), (300, 700), (700, 300),
          (257, 771), (600, 600)]


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()


def _gauss(shapes, seed):
    rng = np.random.default_rng(seed)
    return [torch.from_numpy(rng.standard_normal(sh).astype(np.float32)).to(torch.bfloat16).cuda()
            for sh in shapes]


def _bf(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("coeffs", [oracle.QUINTIC, oracle.CUBIC])
def test_two_e4m3_steps_match_the_oracle(coeffs):
    steps = 5 if coeffs == oracle.QUINTIC else 8
    xs = _gauss(SHAPES, 41)
    f8 = nsa.ns_batched(xs, steps=steps, coeffs=coeffs, fp8_steps=2)
    bf = nsa.ns_batched(xs, steps=steps, coeffs=coeffs)
    torch.cuda.synchronize()
    for x, o8, o16, sh in zip(xs, f8, bf, SHAPES):
        want = oracle.newton_schulz(host_f64(x), steps, coeffs)
        worst = check_blocks(host_f64(o8), want, TOL["bf16"], what=f"e4m3 x2 {sh}")
        e8, e16 = rel_fro(host_f64(o8), want), rel_fro(host_f64(o16), want)
        print(f"  {sh}: e4m3 x2 {e8:.3e} (worst block {worst:.3e}), bf16 {e16:.3e}")
        assert e8 <= 1.1 * e16, (sh, e8, e16)


@pytest.mark.parametrize("nesterov", [False, True])
def test_step_with_e4m3_steps(nesterov):
    """Full step: M' exact to its rounding, the step's own O (read back from a
    step with W = 0) per block against the oracle."""
    import workloads

    shapes = [(300, 700), (700, 300), (1024, 1536), (513, 257)]
    wl = workloads.Workload(name="t", dtype="bf16", shapes=tuple(shapes), call="step", kind="muon",
                            seed=5, nesterov=nesterov)
    ins = device_inputs(wl)
    g = [d["g"] for d in ins]
    wz = [torch.zeros_like(t) for t in g]
    mz = [d["m"].clone() for d in ins]
    nsa.step_batched(wz, g, mz, lr=wl.lr, beta=wl.beta, nesterov=nesterov, steps=5, fp8_steps=2)
    torch.cuda.synchronize()
    for i, (r, c) in enumerate(shapes):
        gh, mh = host_f64(g[i]), host_f64(ins[i]["m"])
        _, m_ref, o_ref = oracle.muon_step(np.zeros_like(gh), gh, mh, lr=wl.lr, beta=wl.beta,
                                           nesterov=nesterov, steps=5)
        assert rel_fro(host_f64(mz[i]), m_ref) <= TOL["bf16"] / 4
        o_step = -host_f64(wz[i]) / (wl.lr * np.sqrt(max(1.0, r / c)))
        check_blocks(o_step, o_ref, TOL["bf16"], what=f"step O {(r, c)}")


def _up(x, a):
    return -(-x // a) * a


def _workspace_f8(ws, shape, which):
    """The e4m3 buffer `which` (0 or 1) of the only matrix of a one-matrix call,
    from the workspace layout (muon_abi.hip): the descriptor table and the
    7 phase prefix arrays, the inverse norm, two sets of 16 tile-claim
    counters, the momentum-pass partials, then X ping, X pong, A, B, and the
    two e4m3 buffers."""
    r, c = shape
    tall = r > c
    sp, lp = _up(min(shape), 256), _up(max(shape), 256)
    off = _up(112, 256) + _up(4 * 7 * 2, 256) + _up(4, 256) + _up(4 * 2 * 16, 256)
    blocks = (sp // 256) * (lp // 64) if tall else (sp // 32) * (lp // 256)
    off += _up(4 * blocks, 256)
    off += 2 * _up(sp * lp * 2, 256) + 2 * _up(sp * sp * 2, 256)
    n = sp * lp
    off += which * _up(n + n // 32, 256)
    raw = ws[off:off + n + n // 32].cpu().numpy()
    return raw[:n], raw[n:], sp, lp


def _decode_f8(data, scales, nrows, ncols):
    """Values of an e4m3 copy in the F8 layout (nrows x ncols)."""
    e4 = torch.from_numpy(data.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    out = np.zeros((nrows, ncols))
    for rr in range(nrows):
        rl = rr % 256
        for cc in range(0, ncols, 32):
            slab = (rr // 256) * (ncols // 64) + cc // 64
            kb = (cc % 64) // 32
            e = int(scales[slab * 512 + 4 * (32 * (2 * (rl // 128) + kb) + rl % 32) + (rl // 32) % 4])
            base = slab * 16384 + rl * 64 + (cc % 64)
            out[rr, cc:cc + 32] = e4[base:base + 32] * 2.0 ** (e - 127)
    return out


@pytest.mark.parametrize("shape", [(700, 300), (300, 700), (512, 1536)])
def test_quantized_transpose_is_exact(shape):
    x = _gauss([shape], 7)[0]
    ws = nsa.allocate_workspace([shape], torch.bfloat16, "cuda", fp8=True)
    nsa.ns_batched([x], steps=2, fp8_steps=1, workspace=ws)
    torch.cuda.synchronize()
    data, scales, sp, lp = _workspace_f8(ws, shape, 1)
    u = host_f64(x)
    u = u.T if shape[0] > shape[1] else u  # the wide orientation: s x l
    xt = np.zeros((lp, sp))
    xt[:u.shape[1], :u.shape[0]] = u.T
    got = _decode_f8(data, scales, lp, sp)
    want = mx_e4m3(xt, 1)
    assert np.array_equal(got, want), int((got != want).sum())


def _emulate(u, steps, fp8_steps, coeffs, eps=1e-7):
    """The e4m3 steps, then bf16 steps, at the library's rounding points, with
    float64 products (the GPU's are fp32 sums, in another order)."""
    a, b, c = coeffs
    tall = u.shape[0] > u.shape[1]
    x = u.T if tall else u
    f = 1.0 / (np.linalg.norm(x) + eps)
    for k in range(steps):
        nf = f if k == 0 else 1.0
        s_g = 1.0 if c != 0 else b
        if k < fp8_steps:
            xq = mx_e4m3(x, 1)
            A = _bf(s_g * nf * nf * (xq @ xq.T))
            aq = mx_e4m3(A, 1)
            if c != 0:
                B = _bf(c * (aq @ aq.T + (b / c) * A))
                bq = mx_e4m3(B, 1)
            else:
                bq = aq
            xtq = mx_e4m3(x.T, 1)
            x = _bf(nf * (bq @ xtq.T + a * x))
        else:
            A = _bf(s_g * nf * nf * (x @ x.T))
            B = _bf(c * (A @ A + (b / c) * A)) if c != 0 else A
            x = _bf(nf * (a * x + B @ x))
    return x.T if tall else x


@pytest.mark.parametrize("coeffs,steps,fp8_steps", [(oracle.QUINTIC, 2, 1),
                                                    ((0.5, 0.25, 0.125), 3, 2),
                                                    (oracle.CUBIC, 3, 2)])
def test_e4m3_steps_against_emulation(coeffs, steps, fp8_steps):
    """Short iterations only: over five quintic steps the polynomial amplifies
    the differences between any two correct implementations (summation order,
    the bf16 roundings they flip) to a few 1e-3, which the oracle test covers."""
    shapes = [(512, 1536), (1536, 512), (300, 700), (600, 600)]
    xs = _gauss(shapes, 3)
    outs = nsa.ns_batched(xs, steps=steps, coeffs=coeffs, fp8_steps=fp8_steps)
    torch.cuda.synchronize()
    for x, o, sh in zip(xs, outs, shapes):
        want = _emulate(host_f64(x), steps, fp8_steps, coeffs)
        worst = float(block_errors(host_f64(o), want).max())
        print(f"  {sh}: worst block against the emulation {worst:.2e}")
        assert worst <= 2e-3, (sh, worst)


def test_e4m3_steps_are_deterministic():
    xs = _gauss([(1024, 3072), (3072, 1024), (300, 700)], 9)
    a = nsa.ns_batched(xs, steps=5, fp8_steps=2)
    b = nsa.ns_batched(xs, steps=5, fp8_steps=2)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))
