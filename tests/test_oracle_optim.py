"""Pins of the oracle's AdamW step (CPU): closed forms of the first step and
of a zero gradient, and torch's own AdamW (fp64, CPU) as an independent
implementation of the same published update."""

import numpy as np
import torch

from oracle import optim

LR, B1, B2, EPS, WD = 2e-4, 0.9, 0.999, 1e-8, 0.01


def test_first_step_moves_each_weight_by_lr_times_the_sign():
    rng = np.random.default_rng(0)
    p = rng.standard_normal(1000)
    g = rng.standard_normal(1000)
    z = np.zeros(1000)
    p1, m1, v1 = optim.adamw_step(p, g, z, z, LR, B1, B2, EPS, 0.0, 1)
    # step 1: m_hat = g, v_hat = g^2, so the update is lr g / (|g| + eps)
    # (the difference of two values near 1 is exact to a few ulp of p)
    assert np.allclose(p - p1, LR * g / (np.abs(g) + EPS), rtol=1e-12, atol=4e-15)
    assert np.allclose(m1, (1 - B1) * g, rtol=1e-15) and np.allclose(v1, (1 - B2) * g * g, rtol=1e-15)


def test_zero_gradient_and_zero_state_only_decay():
    p = np.linspace(-1, 1, 101)
    z = np.zeros_like(p)
    p1, m1, v1 = optim.adamw_step(p, z, z, z, LR, B1, B2, EPS, WD, 7)
    assert np.array_equal(p1, p * (1 - LR * WD))
    assert not m1.any() and not v1.any()


def test_matches_torch_adamw_over_several_steps():
    rng = np.random.default_rng(1)
    p0 = rng.standard_normal((16, 64))
    grads = [rng.standard_normal((16, 64)) * 10.0 ** rng.integers(-4, 1) for _ in range(5)]
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=LR, betas=(B1, B2), eps=EPS, weight_decay=WD)
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = optim.adamw_step(p, g, m, v, LR, B1, B2, EPS, WD, t)
    assert np.allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-15)
    st = opt.state[tp]
    assert np.allclose(m, st["exp_avg"].numpy(), rtol=1e-13)
    assert np.allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13)
