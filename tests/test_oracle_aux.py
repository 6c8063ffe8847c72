"""Pins of the auxiliary-loss and routing-metrics oracle (oracle.aux) to
things other than itself: a hand-worked example, central finite
differences, SciPy's logsumexp, and closed forms of special cases."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "aux_worked_example.json")


def _ev(s):
    return float(eval(s, {"__builtins__": {}}, {"log": math.log, "exp": math.exp, "inf": math.inf}))


def test_worked_example():
    g = json.load(open(GOLDEN))
    lg = np.array([[_ev(v) for v in row] for row in g["logits"]])
    lb, lz = oracle.aux_losses(lg, g["counts"], g["k"])
    assert lb == pytest.approx(_ev(g["L_bal"]), rel=1e-15)
    assert lz == pytest.approx(_ev(g["L_z"]), rel=1e-14)
    np.testing.assert_allclose(oracle.routing_metrics(lg, g["counts"], g["k"]), [_ev(v) for v in g["metrics"]],
                               rtol=1e-14, atol=1e-15)
    for key, (a, b) in (("grad_alpha1_beta0", (1.0, 0.0)), ("grad_alpha0_beta1", (0.0, 1.0))):
        want = np.array([[_ev(v) for v in row] for row in g[key]])
        np.testing.assert_allclose(oracle.aux_losses_grad(lg, g["counts"], g["k"], a, b), want, rtol=1e-14,
                                   atol=1e-16)


def test_gradient_matches_central_differences():
    """Counts are held fixed (they are piecewise constant in the logits)."""
    rng = np.random.default_rng(11)
    T, E, k = 5, 6, 2
    lg = rng.normal(0, 1.5, (T, E))
    counts = np.array([3, 0, 1, 2, 4, 0])
    alpha, beta = 0.7, 0.3

    def obj(z):
        lb, lz = oracle.aux_losses(z, counts, k)
        return alpha * lb + beta * lz

    grad = oracle.aux_losses_grad(lg, counts, k, alpha, beta)
    h = 1e-6
    fd = np.zeros_like(lg)
    for t in range(T):
        for e in range(E):
            zp, zm = lg.copy(), lg.copy()
            zp[t, e] += h
            zm[t, e] -= h
            fd[t, e] = (obj(zp) - obj(zm)) / (2 * h)
    np.testing.assert_allclose(grad, fd, rtol=1e-7, atol=1e-10)


def test_z_loss_against_scipy_logsumexp():
    from scipy.special import logsumexp
    rng = np.random.default_rng(12)
    lg = rng.normal(3.0, 4.0, (50, 9))
    _, lz = oracle.aux_losses(lg, np.full(9, 50 * 2 // 9), 2)
    assert lz == pytest.approx(float(np.mean(logsumexp(lg, axis=1) ** 2)), rel=1e-14)


@pytest.mark.parametrize("E,k,c", [(4, 1, 0.0), (8, 2, -1.5), (64, 8, 3.0)])
def test_even_routing_closed_forms(E, k, c):
    """Equal logits c and even counts: L_bal = 1, L_z = (c + log E)^2,
    entropy log E, max prob 1/E, imbalance 1, zero spread, no balance gradient."""
    T = 2 * E
    lg = np.full((T, E), c)
    counts = np.full(E, T * k // E)
    lb, lz = oracle.aux_losses(lg, counts, k)
    assert lb == pytest.approx(1.0, rel=1e-14)
    assert lz == pytest.approx((c + math.log(E)) ** 2, rel=1e-13, abs=1e-13)
    met = oracle.routing_metrics(lg, counts, k)
    np.testing.assert_allclose(met[:5], [1.0, 0.0, 0.0, math.log(E), 1.0 / E], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.aux_losses_grad(lg, counts, k, 1.0, 0.0), 0.0, atol=1e-17)


def test_collapsed_routing_closed_form():
    """k = 1 and one dominant expert: f = (1, 0, ...), P_0 = 1 / (1 + (E-1) e^-a),
    so L_bal = E P_0; imbalance E; E-1 empty experts."""
    T, E, a = 7, 5, 9.0
    lg = np.zeros((T, E))
    lg[:, 0] = a
    counts = np.array([T, 0, 0, 0, 0])
    lb, _ = oracle.aux_losses(lg, counts, 1)
    assert lb == pytest.approx(E / (1 + (E - 1) * math.exp(-a)), rel=1e-14)
    met = oracle.routing_metrics(lg, counts, 1)
    assert met[0] == pytest.approx(E) and met[1] == E - 1
    assert met[2] == pytest.approx(math.sqrt(E - 1), rel=1e-14)   # std/mean of (T, 0, ..., 0)


def test_count_metrics_by_hand():
    counts = [4, 0, 2, 2]                    # T = 4, k = 2, E = 4: mean 2
    met = oracle.routing_metrics(np.zeros((4, 4)), counts, 2)
    assert met[0] == 2.0 and met[1] == 1.0
    assert met[2] == pytest.approx(math.sqrt(2) / 2, rel=1e-15)
    np.testing.assert_allclose(met[5:9], [0.5, 0.0, 0.25, 0.25])


def test_minus_infinity_logits():
    """-inf logits have p = 0, add nothing to the entropy and keep L_z finite."""
    lg = np.array([[0.0, -np.inf, math.log(3)], [-np.inf, 0.0, 0.0]])
    counts = [0, 1, 1]
    lb, lz = oracle.aux_losses(lg, counts, 1)
    assert math.isfinite(lb) and lz == pytest.approx((math.log(4) ** 2 + math.log(2) ** 2) / 2, rel=1e-14)
    met = oracle.routing_metrics(lg, counts, 1)
    assert met[3] == pytest.approx((math.log(4) - 0.75 * math.log(3) + math.log(2)) / 2, rel=1e-14)
    g = oracle.aux_losses_grad(lg, counts, 1, 1.0, 1.0)
    assert np.all(np.isfinite(g)) and g[0, 1] == 0.0 and g[1, 0] == 0.0


def test_empty_microbatch_contributes_zero():
    """An empty microbatch runs and contributes nothing: adding its losses to
    a per-microbatch sum leaves the sum unchanged; with no tokens every
    expert has zero rows (empty_experts = E) and the token statistics are
    empty sums, reported as 0."""
    rng = np.random.default_rng(5)
    E, k = 6, 2
    lg1 = rng.normal(0, 1, (7, E))
    c1 = np.bincount(np.argsort(-lg1, axis=1, kind="stable")[:, :k].ravel(), minlength=E)
    empty = np.zeros((0, E))
    with_empty = np.add(oracle.aux_losses(lg1, c1, k), oracle.aux_losses(empty, np.zeros(E, int), k))
    assert tuple(with_empty) == oracle.aux_losses(lg1, c1, k)
    m = oracle.routing_metrics(empty, np.zeros(E, int), k)
    assert m.shape == (5 + 2 * E,)
    assert m[1] == E and np.sum(np.zeros(E, int) == 0) == E
    assert np.all(np.delete(m, 1) == 0.0)
