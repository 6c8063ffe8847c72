"""Pins for the oracle's routing and dispatch tables (CPU only).

Each check ties ``oracle.route`` to something other than itself: a
hand-worked example, closed forms, brute-force selection by counting,
invariants of a stable counting sort, and special cases.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from workloads import tie_logits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "route_worked_example.json")


def _ev(s):
    return float(eval(s, {"__builtins__": {}}, {"log": math.log, "exp": math.exp, "inf": math.inf}))


def check_tables(logits, k, r):
    """Invariants that any correct routing + stable dispatch must satisfy."""
    T, E = logits.shape
    ids = r["topk_idx"]
    assert ids.shape == (T, k) and ids.dtype == np.int32
    # k distinct ids per token, all in range
    for t in range(T):
        assert len(set(ids[t].tolist())) == k
        assert ids[t].min() >= 0 and ids[t].max() < E
    # selected logits are in non-increasing order, and every unselected
    # expert loses to the k-th selected one under (logit desc, id asc)
    for t in range(T):
        sel = ids[t]
        for j in range(k - 1):
            a, b = sel[j], sel[j + 1]
            assert logits[t, a] > logits[t, b] or (logits[t, a] == logits[t, b] and a < b)
        last = sel[-1]
        for e in set(range(E)) - set(sel.tolist()):
            assert logits[t, e] < logits[t, last] or (logits[t, e] == logits[t, last] and e > last)
    counts, offsets = r["counts"], r["offsets"]
    assert counts.sum() == T * k
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.all(np.diff(offsets) == counts)
    ros = r["row_of_slot"].reshape(-1)
    sor = r["src_of_row"]
    # bijection and inverse
    assert np.array_equal(np.sort(ros), np.arange(T * k))
    assert np.array_equal(sor[ros], np.arange(T * k))
    flat = ids.reshape(-1)
    for e in range(E):
        seg = sor[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)          # each row sits in its expert's segment
        assert np.all(np.diff(seg) > 0)        # sources ascend inside a segment


def test_worked_example():
    g = json.load(open(GOLDEN))
    logits = np.array([[_ev(v) for v in row] for row in g["logits"]])
    r = oracle.route(logits, g["k"])
    assert r["topk_idx"].tolist() == g["topk_idx"]
    assert r["counts"].tolist() == g["counts"]
    assert r["offsets"].tolist() == g["offsets"]
    assert r["row_of_slot"].tolist() == g["row_of_slot"]
    assert r["src_of_row"].tolist() == g["src_of_row"]
    want = np.array([[_ev(v) for v in row] for row in g["topk_w"]])
    np.testing.assert_allclose(r["topk_w"], want, rtol=1e-14, atol=0)
    rr = oracle.route(logits, g["k"], renorm=True)
    want = np.array([[_ev(v) for v in row] for row in g["topk_w_renorm"]])
    np.testing.assert_allclose(rr["topk_w"], want, rtol=1e-14, atol=0)
    check_tables(logits, g["k"], r)


def test_worked_example_scalar_ffn():
    g = json.load(open(GOLDEN))
    s = g["scalar_ffn"]
    logits = np.array([[_ev(v) for v in row] for row in g["logits"]])
    x = np.array(s["x"])[:, None]
    w_gu = np.array([[[gg], [uu]] for gg, uu in zip(s["gate"], s["up"])])
    w_down = np.array([[[v]] for v in s["down"]])
    out, _ = oracle.layer_fwd(x, w_gu, w_down, g["k"], logits=logits)
    want = np.array([_ev(v) for v in s["out"]])
    np.testing.assert_allclose(out[:, 0], want, rtol=1e-13, atol=1e-15)


def test_softmax_closed_form():
    E = 7
    logits = np.log(np.arange(1, E + 1, dtype=np.float64))[None, :]
    p = oracle.softmax(logits)
    np.testing.assert_allclose(p[0], np.arange(1, E + 1) / (E * (E + 1) / 2), rtol=1e-14)
    r = oracle.route(logits, 3)
    assert r["topk_idx"].tolist() == [[6, 5, 4]]
    np.testing.assert_allclose(r["topk_w"][0], np.array([7, 6, 5]) / 28.0, rtol=1e-14)


@pytest.mark.parametrize("E,k", [(4, 2), (8, 8), (32, 8), (64, 8), (5, 1)])
def test_all_equal_logits(E, k):
    T = 9
    logits = np.full((T, E), 0.25)
    r = oracle.route(logits, k)
    assert np.all(r["topk_idx"] == np.arange(k)[None, :])
    np.testing.assert_allclose(r["topk_w"], 1.0 / E, rtol=1e-15)
    rr = oracle.route(logits, k, renorm=True)
    np.testing.assert_allclose(rr["topk_w"], 1.0 / k, rtol=1e-15)
    assert r["counts"].tolist() == [T] * k + [0] * (E - k)
    # within an expert's segment rows follow token order
    assert r["row_of_slot"][:, 0].tolist() == list(range(T))


def test_k_equals_E_is_full_order():
    rng = np.random.default_rng(0)
    logits = rng.integers(-2, 3, size=(20, 6)).astype(np.float64)
    r = oracle.route(logits, 6)
    for t in range(20):
        want = sorted(range(6), key=lambda e: (-logits[t, e], e))
        assert r["topk_idx"][t].tolist() == want
    np.testing.assert_allclose(r["topk_w"].sum(axis=1), 1.0, rtol=1e-14)


def test_empty_microbatch():
    r = oracle.route(np.zeros((0, 8)), 2)
    assert r["topk_idx"].shape == (0, 2)
    assert r["counts"].tolist() == [0] * 8
    assert r["offsets"].tolist() == [0] * 9
    assert r["src_of_row"].shape == (0,)


def test_nonfinite_order():
    # -inf loses to every finite logit; NaN loses to -inf; +0.0 ties -0.0.
    logits = np.array([[np.nan, -np.inf, 1.0, -0.0, 0.0, np.nan]])
    r = oracle.route(logits, 6)
    assert r["topk_idx"].tolist() == [[2, 3, 4, 1, 0, 5]]
    ids, _ = oracle.route_brute_force(logits, 6)
    assert ids.tolist() == [[2, 3, 4, 1, 0, 5]]


@pytest.mark.parametrize("seed", range(6))
def test_ties_match_brute_force(seed):
    E = [4, 8, 16, 32, 64, 7][seed]
    k = min([2, 8, 3, 8, 8, 7][seed], E)
    logits = tie_logits(24, E, seed, levels=3).astype(np.float64)
    r = oracle.route(logits, k)
    ids, mask = oracle.route_brute_force(logits, k)
    assert np.array_equal(r["topk_idx"], ids)
    check_tables(logits, k, r)


@settings(max_examples=60, deadline=None)
@given(T=st.integers(0, 40), E=st.integers(1, 12), data=st.data())
def test_random_routing_invariants(T, E, data):
    k = data.draw(st.integers(1, E))
    levels = data.draw(st.sampled_from([2, 5, 1000]))
    seed = data.draw(st.integers(0, 2 ** 31 - 1))
    logits = tie_logits(T, E, seed, levels=levels).astype(np.float64)
    r = oracle.route(logits, k)
    check_tables(logits, k, r)
    if T:
        ids, _ = oracle.route_brute_force(logits, k)
        assert np.array_equal(r["topk_idx"], ids)
        p = oracle.softmax(logits)
        np.testing.assert_allclose(r["topk_w"], np.take_along_axis(p, ids.astype(np.int64), 1),
                                   rtol=1e-14)


def test_row_maps_by_counting():
    """row_of_slot[t,j] = offsets[e] + #{(t',j') : id = e, t' < t}, counted
    directly with loops."""
    logits = tie_logits(30, 6, 7, levels=4).astype(np.float64)
    k = 3
    r = oracle.route(logits, k)
    ids = r["topk_idx"]
    for t in range(30):
        for j in range(k):
            e = ids[t, j]
            before = sum(1 for tt in range(t) for jj in range(k) if ids[tt, jj] == e)
            assert r["row_of_slot"][t, j] == r["offsets"][e] + before
