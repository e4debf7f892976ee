"""Parity of the fused AdamW kernel with the float64 oracle, through the C ABI.

Bounds, per element (x' the oracle's float64 result from the same inputs, with
the hyperparameters rounded to float32 as the kernel receives them):
  m, v   a few float32 roundings of each operand: dm = 4 * 2^-24 * (sum of |terms|),
         likewise dv (m' can cancel, so its error is relative to the terms)
  p      float32 evaluation (decay, the update quotient, the subtraction):
         2 ulp32(p') + 8 * 2^-24 * |update| + 2 * 2^-24 * |p|, plus the moments'
         errors carried through the update to first order,
         s * dm / d + s * |m'| * (c * dv / (2 sqrt(v'))) / d^2
         (s = lr / (1 - beta1^t), c = 1 / sqrt(1 - beta2^t), d = c sqrt(v') + eps),
         plus one storage ulp when p is bf16.
"""
import math

import numpy as np
import pytest
import torch

import newton_schulz_03_amd as nsa
import oracle
import workloads
from parity_util import host_f64

pytestmark = pytest.mark.gpu

NUMELS = [1, 7, 8, 9, 255, 8191, 8192, 8193, 100003, 0, 3 * 8192 + 5]
U32 = 2.0 ** -24


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()


def f32(x):
    return float(np.float32(x))


def ulp(x, dtype):
    s = np.spacing(np.abs(x).astype(np.float32)).astype(np.float64)
    return s * (2.0 ** 16 if dtype == "bf16" else 1.0)


def check(dtype, p0, g, m0, v0, p1, m1, v1, kw, step):
    k = {key: f32(val) for key, val in kw.items()}
    pr, mr, vr = oracle.adamw_step(p0, g, m0, v0, step=step, **k)
    bm = 4 * U32 * (k["beta1"] * np.abs(m0) + (1 - k["beta1"]) * np.abs(g)) + 1e-38
    bv = 4 * U32 * (k["beta2"] * v0 + (1 - k["beta2"]) * g * g) + 1e-38
    assert np.all(np.abs(m1 - mr) <= bm), float(np.max(np.abs(m1 - mr) / bm))
    assert np.all(np.abs(v1 - vr) <= bv), float(np.max(np.abs(v1 - vr) / bv))
    upd = np.abs(pr - p0 * (1 - k["lr"] * k["weight_decay"]))
    s_ = k["lr"] / (1 - k["beta1"] ** step)
    c_ = 1 / math.sqrt(1 - k["beta2"] ** step)
    d_ = c_ * np.sqrt(vr) + k["eps"]
    carried = s_ * bm / d_ + s_ * np.abs(mr) * (c_ * bv / (2 * np.sqrt(vr) + 1e-30)) / d_ ** 2
    bp = 2 * ulp(pr, "fp32") + 8 * U32 * upd + 2 * U32 * np.abs(p0) + carried
    if dtype == "bf16":
        bp = bp + ulp(np.maximum(np.abs(pr), np.abs(p1)), "bf16")
    assert np.all(np.abs(p1 - pr) <= bp), float(np.max(np.abs(p1 - pr) / bp))


def make_inputs(dtype, numels, seed):
    wl = workloads.AdamWWorkload(name="t", dtype=dtype, numels=tuple(numels), seed=seed)
    out = []
    for j in range(len(numels)):
        raw = workloads.adamw_inputs(wl, j)
        out.append({"p": workloads.cast(raw["p"], dtype).cuda(),
                    "g": workloads.cast(raw["g"], dtype).cuda(),
                    "m": torch.from_numpy(raw["m"]).cuda(),
                    "v": torch.from_numpy(raw["v"]).cuda()})
    return wl, out


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_adamw_ragged_three_steps(dtype, wd):
    wl, ins = make_inputs(dtype, NUMELS, seed=21)
    kw = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=wd)
    ws = None
    for step in (1, 2, 3):
        if step > 1:  # a fresh gradient for every step
            for j, d in enumerate(ins):
                raw = np.random.default_rng([99, step, j]).standard_normal(NUMELS[j]).astype(np.float32)
                d["g"] = workloads.cast(raw * 1e-3, dtype).cuda()
        before = [{k: host_f64(t) for k, t in d.items()} for d in ins]
        nsa.adamw_batched([d["p"] for d in ins], [d["g"] for d in ins], [d["m"] for d in ins],
                          [d["v"] for d in ins], lr=kw["lr"], betas=(kw["beta1"], kw["beta2"]),
                          eps=kw["eps"], weight_decay=wd, step=step, workspace=ws)
        torch.cuda.synchronize()
        for b, d in zip(before, ins):
            check(dtype, b["p"], b["g"], b["m"], b["v"], host_f64(d["p"]), host_f64(d["m"]),
                  host_f64(d["v"]), kw, step)


def test_adamw_constant_gradient_closed_form_fp32():
    # zero moments and a constant gradient: each step moves p by lr * g / (|g| + eps)
    n = 20000
    g = torch.linspace(-1e-2, 1e-2, n, dtype=torch.float32, device="cuda")
    p = torch.zeros(n, dtype=torch.float32, device="cuda")
    m = torch.zeros_like(p)
    v = torch.zeros_like(p)
    for step in range(1, 6):
        nsa.adamw_batched([p], [g], [m], [v], lr=1e-3, betas=(0.9, 0.95), eps=1e-8,
                          weight_decay=0.0, step=step)
    torch.cuda.synchronize()
    gh = host_f64(g)
    want = -5 * f32(1e-3) * gh / (np.abs(gh) + f32(1e-8))
    assert np.max(np.abs(host_f64(p) - want)) <= 64 * U32 * 5e-3


def test_adamw_full_size_nonexpert_params():
    wl = workloads.adamw_workloads()["adamw_nonexpert_74_layers"]
    ps, gs, ms, vs = [], [], [], []
    for j in range(wl.batch):
        raw = workloads.adamw_inputs(wl, j)
        ps.append(workloads.cast(raw["p"], wl.dtype).cuda())
        gs.append(workloads.cast(raw["g"], wl.dtype).cuda())
        ms.append(torch.from_numpy(raw["m"]).cuda())
        vs.append(torch.from_numpy(raw["v"]).cuda())
    samples = [0, 1, 2, 110, 221, wl.batch - 1]
    before = {j: (host_f64(ps[j]), host_f64(gs[j]), host_f64(ms[j]), host_f64(vs[j])) for j in samples}
    nsa.adamw_batched(ps, gs, ms, vs, lr=wl.lr, betas=(wl.beta1, wl.beta2), eps=wl.eps,
                      weight_decay=wl.weight_decay, step=wl.step)
    torch.cuda.synchronize()
    kw = dict(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps, weight_decay=wl.weight_decay)
    for j in samples:
        p0, g0, m0, v0 = before[j]
        check(wl.dtype, p0, g0, m0, v0, host_f64(ps[j]), host_f64(ms[j]), host_f64(vs[j]), kw,
              wl.step)
    for j in range(wl.batch):
        assert torch.isfinite(ps[j]).all() and torch.isfinite(vs[j]).all(), j
