"""Pins for the oracle's forward and backward (CPU only).

* sparse dropless layer == run-every-expert-then-mask brute force;
* E=1, k=1 reduces to the textbook SwiGLU MLP, evaluated with torch's own
  fp64 ops (a library implementation, not the oracle's code);
* every gradient == torch.autograd of the dense masked formula in fp64, and
  == central finite differences of the oracle's own forward;
* microbatch accumulation: the sum over microbatches equals the
  concatenated batch, and an empty microbatch contributes exactly zero.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import tie_logits


def _problem(T, d, E, k, F, seed, margin=1e-3, x_std=0.5):
    """Random fp64 layer inputs; logits are redrawn until every token's top-k
    margin exceeds ``margin`` so that finite differences cannot flip a
    selection."""
    rng = np.random.default_rng(seed)
    x = rng.normal(0, x_std, (T, d))
    w_gu = rng.normal(0, 0.3, (E, 2 * F, d))
    w_down = rng.normal(0, 0.3, (E, d, F))
    w_router = rng.normal(0, 0.5, (E, d))
    bias = rng.normal(0, 0.1, E)
    for _ in range(1000):
        logits = oracle.router_logits(x, w_router, bias)
        s = -np.sort(-logits, axis=1)
        if k == E or np.min(s[:, k - 1] - s[:, k]) > margin:
            break
        w_router = rng.normal(0, 0.5, (E, d))
    return x, w_gu, w_down, w_router, bias


@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("T,d,E,k,F", [(16, 8, 4, 2, 6), (33, 12, 6, 3, 4), (7, 4, 3, 3, 2), (20, 6, 5, 1, 3)])
def test_sparse_equals_dense_bruteforce(T, d, E, k, F, renorm):
    x, w_gu, w_down, w_router, bias = _problem(T, d, E, k, F, seed=T * 7 + E)
    logits = oracle.router_logits(x, w_router, bias)
    out, _ = oracle.layer_fwd(x, w_gu, w_down, k, logits=logits, renorm=renorm)
    ref = oracle.dense_reference(x, w_gu, w_down, logits, k, renorm=renorm)
    assert np.max(np.abs(out - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_dense_bruteforce_with_ties():
    T, d, E, k, F = 25, 6, 8, 3, 4
    rng = np.random.default_rng(3)
    x = rng.normal(size=(T, d))
    w_gu = rng.normal(size=(E, 2 * F, d))
    w_down = rng.normal(size=(E, d, F))
    logits = tie_logits(T, E, 5, levels=2).astype(np.float64)
    out, _ = oracle.layer_fwd(x, w_gu, w_down, k, logits=logits)
    ref = oracle.dense_reference(x, w_gu, w_down, logits, k)
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_single_expert_is_textbook_swiglu_mlp():
    T, d, F = 11, 16, 24
    rng = np.random.default_rng(1)
    x = rng.normal(size=(T, d))
    w_gu = rng.normal(size=(1, 2 * F, d))
    w_down = rng.normal(size=(1, d, F))
    out, _ = oracle.layer_fwd(x, w_gu, w_down, 1, logits=np.zeros((T, 1)))
    xt = torch.from_numpy(x)
    wg = torch.from_numpy(w_gu[0, :F])
    wu = torch.from_numpy(w_gu[0, F:])
    wd = torch.from_numpy(w_down[0])
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(xt, wg)) * torch.nn.functional.linear(xt, wu), wd)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("renorm", [False, True])
def test_identical_experts_scale_by_weight_sum(renorm):
    T, d, E, k, F = 13, 8, 5, 3, 6
    rng = np.random.default_rng(2)
    x = rng.normal(size=(T, d))
    wg = rng.normal(size=(2 * F, d))
    wd = rng.normal(size=(d, F))
    w_gu = np.repeat(wg[None], E, axis=0)
    w_down = np.repeat(wd[None], E, axis=0)
    logits = rng.normal(size=(T, E))
    out, saved = oracle.layer_fwd(x, w_gu, w_down, k, logits=logits, renorm=renorm)
    h = x @ wg.T
    ffn = (h[:, :F] / (1 + np.exp(-h[:, :F])) * h[:, F:]) @ wd.T
    wsum = saved["topk_w"].sum(axis=1, keepdims=True)
    if renorm:
        np.testing.assert_allclose(wsum, 1.0, rtol=1e-14)
    np.testing.assert_allclose(out, wsum * ffn, rtol=1e-12, atol=1e-12)


def test_token_permutation_equivariance():
    T, d, E, k, F = 19, 8, 6, 2, 5
    x, w_gu, w_down, w_router, bias = _problem(T, d, E, k, F, seed=4)
    logits = oracle.router_logits(x, w_router, bias)
    out, _ = oracle.layer_fwd(x, w_gu, w_down, k, logits=logits)
    perm = np.random.default_rng(9).permutation(T)
    out_p, _ = oracle.layer_fwd(x[perm], w_gu, w_down, k, logits=logits[perm])
    np.testing.assert_allclose(out_p, out[perm], rtol=1e-13, atol=1e-14)


def _torch_dense_grads(x, w_gu, w_down, w_router, bias, k, dout, renorm, logits_given=None):
    """Autograd of the dense masked formula, torch fp64 (library reference)."""
    T, E = x.shape[0], w_gu.shape[0]
    F = w_gu.shape[1] // 2
    xt = torch.tensor(x, requires_grad=True)
    wgu = torch.tensor(w_gu, requires_grad=True)
    wdn = torch.tensor(w_down, requires_grad=True)
    if logits_given is None:
        wr = torch.tensor(w_router, requires_grad=True)
        lg = xt @ wr.T + torch.tensor(bias)
    else:
        wr = None
        lg = torch.tensor(logits_given, requires_grad=True)
    lg.retain_grad()
    with torch.no_grad():
        # selection from the logits' values (piecewise constant)
        order = torch.sort(-lg.detach(), dim=1, stable=True).indices[:, :k]
        mask = torch.zeros(T, E, dtype=torch.bool).scatter_(1, order, True)
    p = torch.softmax(lg, dim=1)
    w = torch.where(mask, p, torch.zeros_like(p))
    if renorm:
        w = w / w.sum(dim=1, keepdim=True)
    out = torch.zeros(T, x.shape[1], dtype=torch.float64)
    for e in range(E):
        h = xt @ wgu[e].T
        y = (torch.nn.functional.silu(h[:, :F]) * h[:, F:]) @ wdn[e].T
        out = out + w[:, e:e + 1] * y
    (out * torch.tensor(dout)).sum().backward()
    g = dict(dx=xt.grad.numpy(), dw_gu=wgu.grad.numpy(), dw_down=wdn.grad.numpy(),
             dlogits=lg.grad.numpy())
    if wr is not None:
        g["dw_router"] = wr.grad.numpy()
    return g


@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("router", [False, True])
@pytest.mark.parametrize("T,d,E,k,F", [(16, 8, 4, 2, 6), (21, 6, 7, 3, 4), (9, 4, 3, 3, 5)])
def test_backward_matches_torch_autograd(T, d, E, k, F, renorm, router):
    x, w_gu, w_down, w_router, bias = _problem(T, d, E, k, F, seed=T + 100 * E + 7 * k)
    dout = np.random.default_rng(5).normal(size=(T, d))
    logits = oracle.router_logits(x, w_router, bias)
    if router:
        out, saved = oracle.layer_fwd(x, w_gu, w_down, k, w_router=w_router, bias=bias, renorm=renorm)
        g = oracle.layer_bwd(dout, saved, w_gu, w_down, x=x, w_router=w_router, renorm=renorm)
        ref = _torch_dense_grads(x, w_gu, w_down, w_router, bias, k, dout, renorm)
    else:
        out, saved = oracle.layer_fwd(x, w_gu, w_down, k, logits=logits, renorm=renorm)
        g = oracle.layer_bwd(dout, saved, w_gu, w_down, renorm=renorm)
        ref = _torch_dense_grads(x, w_gu, w_down, None, None, k, dout, renorm, logits_given=logits)
    for name in ref:
        np.testing.assert_allclose(g[name], ref[name], rtol=1e-10, atol=1e-11, err_msg=name)


def _loss(x, w_gu, w_down, w_router, bias, k, dout, renorm):
    out, _ = oracle.layer_fwd(x, w_gu, w_down, k, w_router=w_router, bias=bias, renorm=renorm)
    return float(np.sum(out * dout))


@pytest.mark.parametrize("renorm", [False, True])
def test_backward_matches_finite_differences(renorm):
    T, d, E, k, F = 12, 6, 4, 2, 5
    x, w_gu, w_down, w_router, bias = _problem(T, d, E, k, F, seed=21, margin=1e-2)
    dout = np.random.default_rng(8).normal(size=(T, d))
    out, saved = oracle.layer_fwd(x, w_gu, w_down, k, w_router=w_router, bias=bias, renorm=renorm)
    g = oracle.layer_bwd(dout, saved, w_gu, w_down, x=x, w_router=w_router, renorm=renorm)
    params = dict(x=x, w_gu=w_gu, w_down=w_down, w_router=w_router)
    grads = dict(x=g["dx"], w_gu=g["dw_gu"], w_down=g["dw_down"], w_router=g["dw_router"])
    rng = np.random.default_rng(11)
    h = 1e-6
    for name, p in params.items():
        # directional derivative along a random direction
        v = rng.normal(size=p.shape)
        args = dict(params)
        args[name] = p + h * v
        lp = _loss(args["x"], args["w_gu"], args["w_down"], args["w_router"], bias, k, dout, renorm)
        args[name] = p - h * v
        lm = _loss(args["x"], args["w_gu"], args["w_down"], args["w_router"], bias, k, dout, renorm)
        fd = (lp - lm) / (2 * h)
        an = float(np.sum(grads[name] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
        # a few individual elements
        flat = p.reshape(-1)
        for idx in rng.choice(flat.size, size=min(25, flat.size), replace=False):
            e = np.zeros_like(flat)
            e[idx] = 1.0
            e = e.reshape(p.shape)
            args[name] = p + h * e
            lp = _loss(args["x"], args["w_gu"], args["w_down"], args["w_router"], bias, k, dout, renorm)
            args[name] = p - h * e
            lm = _loss(args["x"], args["w_gu"], args["w_down"], args["w_router"], bias, k, dout, renorm)
            fd = (lp - lm) / (2 * h)
            an = float(grads[name].reshape(-1)[idx])
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, idx, fd, an)
        args[name] = p


def test_logit_gradient_finite_differences():
    T, d, E, k, F = 10, 5, 6, 3, 4
    x, w_gu, w_down, w_router, bias = _problem(T, d, E, k, F, seed=31, margin=1e-2)
    logits = oracle.router_logits(x, w_router, bias)
    dout = np.random.default_rng(3).normal(size=(T, d))
    for renorm in (False, True):
        out, saved = oracle.layer_fwd(x, w_gu, w_down, k, logits=logits, renorm=renorm)
        g = oracle.layer_bwd(dout, saved, w_gu, w_down, renorm=renorm)
        h = 1e-6
        for t in range(T):
            for e in range(E):
                lp = logits.copy(); lp[t, e] += h
                lm = logits.copy(); lm[t, e] -= h
                fp = np.sum(oracle.layer_fwd(x, w_gu, w_down, k, logits=lp, renorm=renorm)[0] * dout)
                fm = np.sum(oracle.layer_fwd(x, w_gu, w_down, k, logits=lm, renorm=renorm)[0] * dout)
                fd = (fp - fm) / (2 * h)
                assert abs(fd - g["dlogits"][t, e]) <= 1e-7 * max(1.0, abs(fd)), (renorm, t, e)


def test_swiglu_derivative_closed_form():
    z = np.linspace(-8, 8, 97)
    u = np.cos(z) + 2.0
    h = 1e-6
    dg, du = oracle.swiglu_bwd(np.ones_like(z), z, u)
    fd_g = (oracle.silu(z + h) * u - oracle.silu(z - h) * u) / (2 * h)
    np.testing.assert_allclose(dg, fd_g, rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(du, oracle.silu(z), rtol=1e-15)
    # silu'(0) = 1/2, silu(0) = 0
    dg0, du0 = oracle.swiglu_bwd(np.array([1.0]), np.array([0.0]), np.array([1.0]))
    assert dg0[0] == 0.5 and du0[0] == 0.0


def test_sigmoid_extremes():
    s = oracle.sigmoid(np.array([-800.0, -30.0, 0.0, 30.0, 800.0]))
    assert s[0] == 0.0 and s[-1] == 1.0 and s[2] == 0.5
    np.testing.assert_allclose(s[1], np.exp(-30) / (1 + np.exp(-30)), rtol=1e-15)


def test_microbatch_accumulation_equals_concatenation():
    d, E, k, F = 6, 5, 2, 4
    Ts = [9, 0, 14, 3]
    rng = np.random.default_rng(17)
    w_gu = rng.normal(size=(E, 2 * F, d))
    w_down = rng.normal(size=(E, d, F))
    xs = [rng.normal(size=(T, d)) for T in Ts]
    ls = [rng.normal(size=(T, E)) for T in Ts]
    ds = [rng.normal(size=(T, d)) for T in Ts]
    acc_gu = np.zeros_like(w_gu)
    acc_dn = np.zeros_like(w_down)
    for x, l, do in zip(xs, ls, ds):
        out, saved = oracle.layer_fwd(x, w_gu, w_down, k, logits=l)
        g = oracle.layer_bwd(do, saved, w_gu, w_down)
        if x.shape[0] == 0:
            assert np.all(g["dw_gu"] == 0) and np.all(g["dw_down"] == 0)
            assert out.shape == (0, d)
        acc_gu += g["dw_gu"]
        acc_dn += g["dw_down"]
    out, saved = oracle.layer_fwd(np.concatenate(xs), w_gu, w_down, k, logits=np.concatenate(ls))
    g = oracle.layer_bwd(np.concatenate(ds), saved, w_gu, w_down)
    np.testing.assert_allclose(acc_gu, g["dw_gu"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(acc_dn, g["dw_down"], rtol=1e-12, atol=1e-12)


def test_empty_expert_gets_no_rows_and_zero_grads():
    T, d, E, k, F = 15, 6, 5, 2, 4
    rng = np.random.default_rng(2)
    x = rng.normal(size=(T, d))
    w_gu = rng.normal(size=(E, 2 * F, d))
    w_down = rng.normal(size=(E, d, F))
    logits = rng.normal(size=(T, E))
    logits[:, 3] = -1e4
    out, saved = oracle.layer_fwd(x, w_gu, w_down, k, logits=logits)
    assert saved["counts"][3] == 0
    g = oracle.layer_bwd(rng.normal(size=(T, d)), saved, w_gu, w_down)
    assert np.all(g["dw_gu"][3] == 0) and np.all(g["dw_down"][3] == 0)
    assert np.all(g["dlogits"][:, 3] == 0.0)   # p = exp(-1e4 - max) underflows to 0
