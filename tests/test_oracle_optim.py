"""Pins of the AdamW oracle (oracle.optim) to things other than itself:
PyTorch's own AdamW in float64, and closed forms of special cases."""
import numpy as np
import pytest

import oracle


def _torch_adamw(theta0, grads, lr, betas, eps, wd, scale):
    import torch
    p = torch.nn.Parameter(torch.tensor(theta0, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=lr, betas=betas, eps=eps, weight_decay=wd, foreach=False)
    for g in grads:
        p.grad = torch.tensor(g * scale, dtype=torch.float64)
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("wd,scale", [(0.0, 1.0), (0.1, 1.0), (0.01, 0.25)])
def test_matches_torch_adamw_float64(wd, scale):
    rng = np.random.default_rng(7)
    n = 257
    theta = rng.normal(0, 0.02, n)
    grads = [rng.normal(0, 1e-3, n) * (1 + i) for i in range(6)]
    grads[2][::7] = 0.0          # exactly zero gradients on some elements
    lr, betas, eps = 3e-3, (0.9, 0.95), 1e-8
    m = np.zeros(n)
    v = np.zeros(n)
    th = theta.copy()
    for t, g in enumerate(grads, start=1):
        th, m, v = oracle.adamw_step(th, g, m, v, t, lr, betas[0], betas[1], eps, wd, grad_scale=scale)
    ref = _torch_adamw(theta, grads, lr, betas, eps, wd, scale)
    for got, want in zip((th, m, v), ref):
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-18)


def test_constant_gradient_closed_form():
    """lambda = 0, m = v = 0 at the start, the same g every step: the bias
    corrections make m_hat = g and v_hat = g^2 exactly, so each step moves
    theta by lr * g / (|g| + eps)."""
    g = np.array([1e-3, -2.5e-2, 4.0, -1e-6])
    theta0 = np.array([0.5, -0.25, 0.0, 1.0])
    lr, eps = 1e-2, 1e-8
    th, m, v = theta0.copy(), np.zeros(4), np.zeros(4)
    for t in range(1, 11):
        th, m, v = oracle.adamw_step(th, g, m, v, t, lr, 0.9, 0.999, eps, 0.0)
        np.testing.assert_allclose(m / (1 - 0.9 ** t), g, rtol=1e-13)
        np.testing.assert_allclose(v / (1 - 0.999 ** t), g * g, rtol=1e-12)
        np.testing.assert_allclose(th, theta0 - t * lr * g / (np.abs(g) + eps), rtol=1e-12, atol=1e-15)


def test_zero_gradient_pure_decay():
    """g = 0: the moments stay zero and theta shrinks by (1 - lr*lambda) per step."""
    theta0 = np.linspace(-1, 1, 9)
    lr, wd = 1e-3, 0.1
    th, m, v = theta0.copy(), np.zeros(9), np.zeros(9)
    for t in range(1, 6):
        th, m, v = oracle.adamw_step(th, np.zeros(9), m, v, t, lr, weight_decay=wd)
        assert np.all(m == 0) and np.all(v == 0)
        np.testing.assert_allclose(th, theta0 * (1 - lr * wd) ** t, rtol=1e-14)


def test_first_step_closed_form_with_decay():
    theta0 = np.array([0.3, -0.7])
    g = np.array([2e-4, 5e-2])
    lr, wd, eps = 1e-3, 0.05, 1e-6
    th, m, v = oracle.adamw_step(theta0, g, np.zeros(2), np.zeros(2), 1, lr, 0.8, 0.99, eps, wd)
    np.testing.assert_allclose(m, 0.2 * g, rtol=1e-15)
    np.testing.assert_allclose(v, 0.01 * g * g, rtol=1e-14)
    np.testing.assert_allclose(th, theta0 * (1 - lr * wd) - lr * g / (np.abs(g) + eps), rtol=1e-14)


def test_grad_scale_is_a_plain_product():
    rng = np.random.default_rng(3)
    th, g = rng.normal(size=16), rng.normal(size=16)
    a = oracle.adamw_step(th, g, np.zeros(16), np.zeros(16), 1, 1e-3, grad_scale=0.5)
    b = oracle.adamw_step(th, 0.5 * g, np.zeros(16), np.zeros(16), 1, 1e-3)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_step_number_starts_at_one():
    with pytest.raises(ValueError):
        oracle.adamw_step(np.zeros(2), np.zeros(2), np.zeros(2), np.zeros(2), 0, 1e-3)
