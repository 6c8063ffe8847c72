"""Pins of the expert-parallel exchange oracle (oracle.ep), CPU only:

* a hand-worked two-rank example (tests/golden/ep_worked_example.json) with
  uneven sources and an empty source: send tables, received counts, receive
  plans and regroup maps;
* invariants of the receive plan on random tables: regroup_row is a bijection,
  each local expert's rows are contiguous with sources in order and each
  source's rows in their segment order;
* the whole exchange is a permutation of rows, so every source's outputs and
  token gradients equal those of the single-rank layer over all EP*E_local
  experts (oracle.moe, itself pinned to brute force and autograd), and every
  expert's weight gradient equals the sum over sources of the single-rank
  gradients; checked with uneven sources, an empty source and empty experts.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ep_worked_example.json")


def _routes(logit_list, k):
    return [oracle.route(np.asarray(l, dtype=np.float64), k) if len(l) else None for l in logit_list]


@pytest.mark.parametrize("case", ["uneven", "empty_source"])
def test_worked_example(case):
    g = json.load(open(GOLDEN))
    ep, e_local, k = g["ep"], g["e_local"], g["k"]
    logits = [g["logits"]["source0"], g["logits"]["source1"] if case == "uneven" else []]
    want = g[case]
    plans_s = []
    for s, l in enumerate(logits):
        if len(l):
            r = oracle.route(np.asarray(l, dtype=np.float64), k)
            sc, so = oracle.ep_send_plan(r["counts"], r["offsets"], ep, len(l))
        else:
            sc, so = oracle.ep_send_plan(np.zeros(ep * e_local, np.int32), None, ep, 0)
        assert sc.tolist() == want["send_counts"][s], (case, s)
        assert so.tolist() == want["send_offsets"][s], (case, s)
        plans_s.append(sc)
    for r in range(ep):
        rc = np.stack([plans_s[s][r] for s in range(ep)])
        assert rc.tolist() == want["recv_counts"][r]
        p = oracle.ep_recv_plan(rc)
        for key in ("local_counts", "local_offsets", "recv_offsets", "regroup_row"):
            assert p[key].tolist() == want[key][r], (case, r, key)


def test_recv_plan_invariants():
    rng = np.random.default_rng(4)
    for trial in range(200):
        ep = int(rng.integers(1, 9))
        e_local = int(rng.integers(1, 17))
        rc = rng.integers(0, 6, size=(ep, e_local))
        rc[rng.random((ep, e_local)) < 0.3] = 0
        if trial % 7 == 0:
            rc[int(rng.integers(0, ep))] = 0          # an empty source
        if trial % 5 == 0:
            rc[:, int(rng.integers(0, e_local))] = 0  # an empty local expert
        p = oracle.ep_recv_plan(rc)
        R = int(rc.sum())
        g = p["regroup_row"]
        assert sorted(g.tolist()) == list(range(R))
        assert p["local_offsets"][-1] == R and p["recv_offsets"][-1] == R
        assert np.array_equal(p["local_counts"], rc.sum(axis=0))
        # walk the received rows by hand: source-major, local expert inside
        i = 0
        seen = {e: [] for e in range(e_local)}
        for s in range(ep):
            assert p["recv_offsets"][s] == i
            for e in range(e_local):
                for _ in range(rc[s, e]):
                    seen[e].append((s, i, int(g[i])))
                    i += 1
        for e in range(e_local):
            rows = [gr for _, _, gr in seen[e]]
            # contiguous in [local_offsets[e], local_offsets[e+1]), sources in order, received order kept
            assert rows == list(range(p["local_offsets"][e], p["local_offsets"][e + 1]))


def _problem(Ts, d, E, k, F, seed):
    rng = np.random.default_rng(seed)
    xs = [rng.normal(0, 0.5, (T, d)) for T in Ts]
    logits = [rng.normal(0, 1.0, (T, E)) for T in Ts]
    w_gu = rng.normal(0, 0.3, (E, 2 * F, d))
    w_down = rng.normal(0, 0.3, (E, d, F))
    douts = [rng.normal(0, 1.0, (T, d)) for T in Ts]
    return xs, logits, w_gu, w_down, douts


@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("Ts,ep,e_local,k", [((9, 4), 2, 3, 2), ((7, 0, 11), 3, 2, 3), ((0, 5), 2, 4, 1),
                                           ((6, 6, 2, 9), 4, 2, 4), ((13,), 1, 5, 2)])
def test_exchange_equals_single_rank_layer(Ts, ep, e_local, k, renorm):
    d, F = 6, 4
    E = ep * e_local
    xs, logits, w_gu, w_down, douts = _problem(Ts, d, E, k, F, seed=sum(Ts) * 13 + ep)
    if ep > 1 and Ts[0] > 0:  # one global expert nobody picks: an empty local expert somewhere
        for l in logits:
            l[:, E - 1] = -50.0
    outs, saved = oracle.ep_layer_fwd(xs, logits, w_gu, w_down, k, ep, renorm)
    g = oracle.ep_layer_bwd(douts, saved, w_gu, w_down)
    dw_gu = np.zeros_like(w_gu)
    dw_down = np.zeros_like(w_down)
    for s, T in enumerate(Ts):
        if T == 0:
            assert outs[s].shape == (0, d) and g["dx"][s].shape == (0, d)
            assert not saved["send_counts"][s].any() and not saved["send_offsets"][s].any()
            continue
        out_ref, sv = oracle.layer_fwd(xs[s], w_gu, w_down, k, logits=logits[s], renorm=renorm)
        gr = oracle.layer_bwd(douts[s], sv, w_gu, w_down, renorm=renorm)
        np.testing.assert_allclose(outs[s], out_ref, rtol=1e-12, atol=1e-13)
        for key in ("dx", "dlogits", "dtopk_w", "dy", "dx_perm"):
            np.testing.assert_allclose(g[key][s], gr[key], rtol=1e-12, atol=1e-13, err_msg=key)
        dw_gu += gr["dw_gu"]
        dw_down += gr["dw_down"]
    np.testing.assert_allclose(g["dw_gu"], dw_gu, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["dw_down"], dw_down, rtol=1e-12, atol=1e-13)
    # every destination got exactly the rows routed to its experts
    for r in range(ep):
        want = sum(int(sv["counts"][r * e_local:(r + 1) * e_local].sum())
                   for sv in saved["routes"] if sv is not None)
        assert saved["plans"][r]["recv_offsets"][-1] == want
