"""Pins of the float64 AdamW oracle.

- torch.optim.AdamW (a library implementation) on the same float64 tensors,
  over several steps;
- closed forms:
  - with a constant gradient and zero initial moments, the bias-corrected
    moments are g and g^2 at every step, so each step moves p by
    lr * g / (|g| + eps) (weight decay 0);
  - a zero gradient on zero moments leaves only the decay p * (1 - lr * wd);
- planted mistakes in a copy of the update must fail one of the pins.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

KW = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def torch_adamw(p, g_seq, kw):
    t = torch.tensor(p, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([t], lr=kw["lr"], betas=(kw["beta1"], kw["beta2"]), eps=kw["eps"],
                            weight_decay=kw["weight_decay"], foreach=False, fused=False)
    for g in g_seq:
        t.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
    st = opt.state[t]
    return t.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


def run_oracle(p, g_seq, kw, step_fn=None):
    step_fn = step_fn or oracle.adamw_step
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    for t, g in enumerate(g_seq, start=1):
        p, m, v = step_fn(p, g, m, v, step=t, **kw)
    return p, m, v


def cases():
    rng = np.random.default_rng(11)
    p = rng.standard_normal(257) * 0.02
    gs = [rng.standard_normal(257) * 1e-3 for _ in range(6)]
    return p, gs


def test_matches_torch_adamw_over_steps():
    p, gs = cases()
    for kw in (KW, dict(KW, weight_decay=0.0), dict(KW, beta1=0.0, beta2=0.5, eps=1e-3)):
        want = torch_adamw(p, gs, kw)
        got = run_oracle(p, gs, kw)
        for a, b in zip(got, want):
            np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-16)


def test_constant_gradient_closed_form():
    rng = np.random.default_rng(12)
    p = rng.standard_normal(64)
    g = rng.standard_normal(64) * 1e-2
    kw = dict(KW, weight_decay=0.0)
    steps = 7
    got, m, v = run_oracle(p, [g] * steps, kw)
    want = p - steps * kw["lr"] * g / (np.abs(g) + kw["eps"])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)
    np.testing.assert_allclose(m, (1 - kw["beta1"] ** steps) * g, rtol=1e-14)
    np.testing.assert_allclose(v, (1 - kw["beta2"] ** steps) * g * g, rtol=1e-14)


def test_zero_gradient_is_pure_decay():
    p = np.linspace(-1, 1, 33)
    z = np.zeros_like(p)
    got, m, v = oracle.adamw_step(p, z, z, z, step=3, **KW)
    np.testing.assert_array_equal(m, 0.0)
    np.testing.assert_array_equal(v, 0.0)
    np.testing.assert_allclose(got, p * (1 - KW["lr"] * KW["weight_decay"]), rtol=1e-15)


def _mutant(kind):
    def step(p, g, m, v, lr, beta1, beta2, eps, weight_decay, step):
        p = np.asarray(p, np.float64)
        if kind != "no_decay":
            p = p * (1.0 - lr * weight_decay)
        m = beta1 * m + (1.0 - beta1) * g
        v = beta2 * v + (1.0 - beta2) * (g if kind == "v_linear" else g * g)
        bc1 = 1.0 - beta1 ** (step if kind != "bias_t_minus_1" else max(step - 1, 1))
        bc2 = 1.0 - beta2 ** step
        denom = np.sqrt(v / bc2) + eps if kind != "eps_inside" else np.sqrt(v / bc2 + eps)
        p = p - lr * (m / bc1) / denom
        return p, m, v
    return step


@pytest.mark.parametrize("kind", ["no_decay", "v_linear", "bias_t_minus_1", "eps_inside"])
def test_planted_adamw_mistake_fails_a_pin(kind):
    p, gs = cases()
    gs = [np.abs(g) for g in gs] if kind == "v_linear" else gs
    want = torch_adamw(p, gs, KW)
    got = run_oracle(p, gs, KW, step_fn=_mutant(kind))
    assert any(not np.allclose(a, b, rtol=1e-9, atol=1e-12) for a, b in zip(got, want))


def test_adamw_workload_shapes():
    wl = workloads.adamw_workloads()["adamw_nonexpert_74_layers"]
    assert wl.batch == 74 * 3 + 1
    assert sum(wl.numels) == 74 * (2 * 6144 + 384 * 6144) + 6144
    ins = workloads.adamw_inputs(wl, 2)
    assert ins["p"].shape == (384 * 6144,) and (ins["v"] >= 0).all()
