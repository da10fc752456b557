"""Pins for the oracle's adapter optimizer step (Adam, decoupled weight decay).

Pinned by:
  * closed forms: the first step from zero moments moves each weight by
    lr g / (|g| + eps) (plus the decay), and a zero gradient only decays;
  * torch.optim.AdamW, an independent implementation of the same textbook
    step, run in float64 over several steps with the same hyperparameters.
"""

import numpy as np
import torch

from oracle import qlora_oracle as O


def test_first_step_closed_form():
    rng = np.random.default_rng(1)
    p = rng.standard_normal(1000)
    g = rng.standard_normal(1000)
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.999, 1e-8, 0.01
    p1, m1, v1 = O.adam_step(p, g, np.zeros_like(p), np.zeros_like(p), 1, lr, b1, b2, eps, wd)
    assert np.allclose(m1, 0.1 * g, rtol=1e-15, atol=0)
    assert np.allclose(v1, 0.001 * g * g, rtol=1e-14, atol=0)
    want = p * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
    assert np.allclose(p1, want, rtol=1e-13, atol=1e-16)


def test_zero_gradient_only_decays():
    p = np.linspace(-1, 1, 101)
    p1, m1, v1 = O.adam_step(p, np.zeros_like(p), np.zeros_like(p), np.zeros_like(p), 3, 1e-2, 0.9, 0.99, 1e-8, 0.1)
    assert np.array_equal(m1, np.zeros_like(p)) and np.array_equal(v1, np.zeros_like(p))
    assert np.allclose(p1, p * (1 - 1e-3), rtol=1e-15, atol=0)


def test_matches_torch_adamw_float64_over_steps():
    rng = np.random.default_rng(7)
    n = 777
    p0 = rng.standard_normal(n)
    grads = [rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 1) for _ in range(5)]
    lr, b1, b2, eps, wd = 2e-4, 0.9, 0.999, 1e-8, 0.05
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = O.adam_step(p, g, m, v, t, lr, b1, b2, eps, wd)
        assert np.allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-15), t
    st = opt.state[tp]
    assert np.allclose(m, st["exp_avg"].numpy(), rtol=1e-13, atol=0)
    assert np.allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13, atol=0)
