"""Pins of the AdamW oracle (oracle/adamw.py) against closed forms and an independent
implementation; CPU only."""

import numpy as np
import pytest
import torch

from oracle import adamw as oa


def test_first_step_closed_form():
    """From m = v = 0 the bias-corrected moments are g and g^2, so the step is
    W (1 - lr wd) - lr g / (|g| + eps)."""
    rng = np.random.default_rng(1)
    W, G = rng.standard_normal(1000), rng.standard_normal(1000) * 1e-3
    lr, wd, eps = 3e-3, 0.1, 1e-8
    W1, m1, v1 = oa.adamw_step(W, G, np.zeros(1000), np.zeros(1000), 1, lr=lr, wd=wd, eps=eps)
    assert np.allclose(W1, W * (1 - lr * wd) - lr * G / (np.abs(G) + eps), rtol=1e-13, atol=0)
    assert np.allclose(m1, 0.1 * G, rtol=1e-15) and np.allclose(v1, 0.001 * G * G, rtol=1e-15)


def test_constant_gradient_geometric_series():
    """With a constant gradient the moments are g (1 - beta1^t) and g^2 (1 - beta2^t), so
    every bias-corrected step is lr g / (|g| + eps) whatever t."""
    g = np.array([2.0, -0.5, 1e-3, 0.0])
    W = np.array([1.0, 1.0, 1.0, 1.0])
    m = v = np.zeros(4)
    b1, b2, lr, eps = 0.9, 0.99, 0.01, 1e-8
    for t in range(1, 8):
        W_prev = W
        W, m, v = oa.adamw_step(W, g, m, v, t, lr=lr, beta1=b1, beta2=b2, eps=eps)
        assert np.allclose(m, g * (1 - b1 ** t), rtol=1e-13)
        assert np.allclose(v, g * g * (1 - b2 ** t), rtol=1e-13)
        assert np.allclose(W_prev - W, lr * g / (np.abs(g) + eps), rtol=1e-9, atol=1e-18)


@pytest.mark.parametrize("wd", [0.0, 0.05])
def test_matches_torch_adamw(wd):
    """torch.optim.AdamW (float64, CPU) over 6 steps with changing gradients."""
    rng = np.random.default_rng(7)
    W0 = rng.standard_normal((37, 5))
    p = torch.nn.Parameter(torch.from_numpy(W0.copy()))
    opt = torch.optim.AdamW([p], lr=2e-3, betas=(0.9, 0.95), eps=1e-6, weight_decay=wd)
    W, m, v = W0.copy(), np.zeros_like(W0), np.zeros_like(W0)
    for t in range(1, 7):
        G = rng.standard_normal(W0.shape) * (0.1 * t)
        p.grad = torch.from_numpy(G.copy())
        opt.step()
        W, m, v = oa.adamw_step(W, G, m, v, t, lr=2e-3, beta1=0.9, beta2=0.95, eps=1e-6, wd=wd)
        assert np.allclose(W, p.detach().numpy(), rtol=1e-12, atol=1e-14)


def test_planted_mistakes_fail_a_pin():
    """A missing bias correction or decay applied after the step changes the first step."""
    rng = np.random.default_rng(3)
    W, G = rng.standard_normal(50), rng.standard_normal(50)
    lr, wd = 1e-2, 0.3
    good, _, _ = oa.adamw_step(W, G, np.zeros(50), np.zeros(50), 1, lr=lr, wd=wd)
    no_bc = W * (1 - lr * wd) - lr * (0.1 * G) / (np.sqrt(0.001 * G * G) + 1e-8)
    decay_after = (W - lr * G / (np.abs(G) + 1e-8)) * (1 - lr * wd)
    assert not np.allclose(good, no_bc) and not np.allclose(good, decay_after)
    with pytest.raises(ValueError):
        oa.adamw_step(W, G, np.zeros(50), np.zeros(50), 0)
