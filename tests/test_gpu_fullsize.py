"""Parity at full workload sizes, in the launch configuration the bench times.

The layer is per token and per expert, so the fp64 oracle can be streamed
one expert at a time: expert e's rows of every saved tensor and its weight
gradients depend only on its own rows, and the token-side results are sums
over the experts of each token.

  * ep_share_32k (T=32768, d=2048, E=32, k=8, F=1408) is compared in FULL:
    the routing and dispatch tables bit for bit; x_perm bit for bit; every
    expert's rows of h, a, y, dy, dh and dx_perm; every expert's dw_gu and
    dw_down (the heaviest, with ~32k rows, included; empty experts exactly
    zero); out, dx, dtopk_w and dlogits for every token.
  * large_share_uniform (d=4096, E=64, F=1536) is compared in full the same
    way (every expert's rows and weight gradients, every token).
  * large_share_zipf / large_share_uniform: the tables bit for bit, sampled
    dispatched rows bit for bit, sampled tokens' outputs and token-side
    gradients, and the full weight gradients of the heaviest, a median and the
    lightest expert.
  * microbatches_32k (T = 16384, 7001, 0, 32768 on one set of buffers): each
    microbatch's tables bit for bit and sampled tokens, then the accumulated
    weight gradients of the heaviest and the lightest expert that is live in
    every non-empty microbatch; the empty microbatch leaves dW bit-identical.

Bars: max|gpu - ref| / max|ref| <= 2e-2 per expert slice (bf16 layer),
routing weights 1e-4; where max|ref| = 0 the GPU value must be exactly 0.
"""
import numpy as np
import pytest

import oracle
from tests.parity_util import TOL, TOL_ROUTING, assert_close, to_device, to_host64
from workloads import BF16, F32, WORKLOADS, make_inputs, to_f64

pytestmark = pytest.mark.gpu


def _run_full(w, inp, recompute=False):
    import torch
    import token_dispatch_grouped_amd as moe
    from token_dispatch_grouped_amd.layer import MoeLayer
    mb = inp["micro"][0]
    W = inp["weights"]
    T = mb["x"].shape[0]
    layer = MoeLayer(T, w.d, w.E, w.k, w.F, moe.MOE_DTYPE_BF16, recompute=recompute)
    x = to_device(mb["x"], BF16)
    dout = to_device(mb["dout"], BF16)
    wgu = to_device(W["w_gu"], BF16)
    wdn = to_device(W["w_down"], BF16)
    lg = to_device(mb["logits"], F32)
    dw_gu = torch.zeros(w.E, 2 * w.F, w.d, device="cuda")
    dw_dn = torch.zeros(w.E, w.d, w.F, device="cuda")
    sv = layer.forward(T, x, wgu, wdn, logits=lg)
    g = layer.backward(T, dout, wgu, wdn, dw_gu, dw_dn)
    torch.cuda.synchronize()
    return layer, sv, g, dw_gu, dw_dn


def _expert_oracle(e, r, k, x64, dout64, w_gu_bits, w_down_bits):
    """fp64 oracle of expert e alone, on its own rows [offsets[e], offsets[e+1]):
    the forward (h, a, y), the combine backward's dy for those rows and the
    FFN backward (dh, dx rows, dw_gu, dw_down). Returns None for an empty
    expert."""
    lo, hi = int(r["offsets"][e]), int(r["offsets"][e + 1])
    if hi == lo:
        return None
    slots = r["src_of_row"][lo:hi]
    t_of = slots // k
    wgu = to_f64(w_gu_bits[e:e + 1], BF16)
    wdn = to_f64(w_down_bits[e:e + 1], BF16)
    x_e = x64[t_of]
    off1 = np.array([0, hi - lo], dtype=np.int32)
    h, a, y = oracle.expert_ffn_fwd(x_e, wgu, wdn, off1)
    w_e = r["topk_w"].reshape(-1)[slots][:, None]
    dy, dtw = oracle.unpermute_combine_bwd(dout64[t_of], y, w_e, np.arange(hi - lo, dtype=np.int32)[:, None])
    dx, dwgu, dwdn, dh = oracle.expert_ffn_bwd(dy, x_e, h, a, wgu, wdn, off1)
    return dict(lo=lo, hi=hi, slots=slots, t_of=t_of, w=w_e, h=h, a=a, y=y, dy=dy, dtw=dtw[:, 0], dh=dh, dx=dx,
                dw_gu=dwgu[0], dw_down=dwdn[0])


def _check_tables(sv, r, n_empty):
    for key in ("topk_idx", "counts", "offsets", "row_of_slot", "src_of_row"):
        assert np.array_equal(getattr(sv, key).cpu().numpy(), r[key]), key
    assert_close("topk_w", to_host64(sv.topk_w), r["topk_w"], TOL_ROUTING)
    assert int((r["counts"] == 0).sum()) == n_empty


def _check_dw(e, o, dw_gu, dw_dn, tol):
    assert_close(f"dw_gu[{e}]", to_host64(dw_gu[e]), o["dw_gu"], tol)
    assert_close(f"dw_down[{e}]", to_host64(dw_dn[e]), o["dw_down"], tol)


@pytest.mark.parametrize("name", ["ep_share_32k", "large_share_uniform"])
def test_fullsize_every_expert(name):
    """The bench workload, and the d = 4096 share with uniform routing,
    compared in full, one expert at a time."""
    import torch
    w = WORKLOADS[name]
    print(f"[fullsize] every expert {w.name}: T={w.T} d={w.d} E={w.E} k={w.k} F={w.F}", flush=True)
    inp = make_inputs(w)
    mb, W = inp["micro"][0], inp["weights"]
    T, k, tol = w.T, w.k, TOL[BF16]
    layer, sv, g, dw_gu, dw_dn = _run_full(w, inp)
    r = oracle.route(mb["logits"].astype(np.float64), k)
    _check_tables(sv, r, w.n_empty)
    x64, dout64 = to_f64(mb["x"], BF16), to_f64(mb["dout"], BF16)
    assert np.array_equal(to_host64(sv.x_perm), x64[r["src_of_row"] // k]), "x_perm"

    # token-side results are sums over a token's experts, accumulated as the
    # experts are visited (a token picks an expert at most once, so the row
    # indices of one expert are distinct)
    out = np.zeros((T, w.d))
    dx = np.zeros((T, w.d))
    dtw = np.zeros(T * k)
    for e in range(w.E):
        o = _expert_oracle(e, r, k, x64, dout64, W["w_gu"], W["w_down"])
        if o is None:
            assert float(dw_gu[e].abs().max()) == 0.0 and float(dw_dn[e].abs().max()) == 0.0, e
            continue
        lo, hi = o["lo"], o["hi"]
        print(f"[fullsize] expert {e}: {hi - lo} rows", flush=True)
        for key, gpu_t in (("h", sv.h), ("a", sv.a), ("y", sv.y), ("dy", g["dy"]), ("dh", g["dh"]),
                           ("dx", g["dx_perm"])):
            assert_close(f"{key}[expert {e}]", to_host64(gpu_t[lo:hi]), o[key], tol)
        _check_dw(e, o, dw_gu, dw_dn, tol)
        out[o["t_of"]] += o["w"] * o["y"]
        dx[o["t_of"]] += o["dx"]
        dtw[o["slots"]] = o["dtw"]
    dtw = dtw.reshape(T, k)
    assert_close("out", to_host64(sv.out), out, tol)
    assert_close("dx", to_host64(g["dx"]), dx, tol)
    assert_close("dtopk_w", to_host64(g["dtopk_w"]), dtw, tol)
    dlogits = oracle.route_bwd(dtw, mb["logits"].astype(np.float64), r["topk_idx"], r["topk_w"])
    assert_close("dlogits", to_host64(g["dlogits"]), dlogits, tol)
    for t in (sv.out, sv.y, sv.h, g["dx"], g["dx_perm"], dw_gu, dw_dn):
        assert bool(torch.isfinite(t).all())


@pytest.mark.parametrize("name", ["large_share_zipf", "large_share_uniform"])
def test_fullsize_sampled_large_share(name):
    w = WORKLOADS[name]
    print(f"[fullsize] {name}: T={w.T} d={w.d} E={w.E} k={w.k} F={w.F}", flush=True)
    inp = make_inputs(w)
    mb, W = inp["micro"][0], inp["weights"]
    T, k, tol = w.T, w.k, TOL[BF16]
    layer, sv, g, dw_gu, dw_dn = _run_full(w, inp)
    r = oracle.route(mb["logits"].astype(np.float64), k)
    _check_tables(sv, r, w.n_empty)
    counts = r["counts"]

    # --- dispatched copy on sampled rows, bit-exact
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.integers(0, T * k, 4000), [0, T * k - 1]]))
    xp = to_host64(sv.x_perm[rows.tolist()])
    want = to_f64(mb["x"], BF16)[r["src_of_row"][rows] // k]
    assert np.array_equal(xp, want), "x_perm rows"

    # --- sampled tokens: forward outputs and token-side gradients (the oracle
    # on the sub-batch of sampled tokens gives exactly those tokens' results)
    toks = np.unique(np.concatenate([rng.integers(0, T, 40), [0, T - 1]]))
    wgu64, wdn64 = to_f64(W["w_gu"], BF16), to_f64(W["w_down"], BF16)
    xs = to_f64(mb["x"], BF16)[toks]
    ds = to_f64(mb["dout"], BF16)[toks]
    out_s, sv_s = oracle.layer_fwd(xs, wgu64, wdn64, k, logits=mb["logits"][toks].astype(np.float64))
    g_s = oracle.layer_bwd(ds, sv_s, wgu64, wdn64)
    del wgu64, wdn64
    assert_close("out", to_host64(sv.out[toks.tolist()]), out_s, tol)
    assert_close("dx", to_host64(g["dx"][toks.tolist()]), g_s["dx"], tol)
    assert_close("dtopk_w", to_host64(g["dtopk_w"][toks.tolist()]), g_s["dtopk_w"], tol)
    assert_close("dlogits", to_host64(g["dlogits"][toks.tolist()]), g_s["dlogits"], tol)
    full_rows = r["row_of_slot"][toks].reshape(-1)
    sub_rows = sv_s["row_of_slot"].reshape(-1)
    for key, gpu_t in (("h", sv.h), ("a", sv.a), ("y", sv.y), ("dy", g["dy"]), ("dx_perm", g["dx_perm"]),
                       ("dh", g["dh"])):
        ref = (sv_s if key in ("h", "a", "y") else g_s)[key][sub_rows]
        assert_close(key, to_host64(gpu_t[full_rows.tolist()]), ref, tol)

    # --- full weight gradients of the heaviest, a median and the lightest expert
    live = np.nonzero(counts > 0)[0]
    by_rows = live[np.argsort(counts[live], kind="stable")]
    picks = sorted({int(by_rows[-1]), int(by_rows[len(by_rows) // 2]), int(by_rows[0])})
    x64, dout64 = to_f64(mb["x"], BF16), to_f64(mb["dout"], BF16)
    for e in picks:
        print(f"[fullsize] dW check on expert {e} with {counts[e]} rows", flush=True)
        o = _expert_oracle(e, r, k, x64, dout64, W["w_gu"], W["w_down"])
        _check_dw(e, o, dw_gu, dw_dn, tol)
    for ee in np.nonzero(counts == 0)[0]:
        assert float(dw_gu[int(ee)].abs().max()) == 0.0 and float(dw_dn[int(ee)].abs().max()) == 0.0
    import torch
    for t in (sv.out, sv.y, sv.h, g["dx"], g["dx_perm"], dw_gu, dw_dn):
        assert bool(torch.isfinite(t).all())


def test_fullsize_microbatch_accumulation():
    """Four microbatches T = 16384, 7001, 0, 32768 on one set of buffers sized
    for the largest; fp32 weight gradients accumulate; the empty microbatch
    launches nothing and leaves them bit-identical."""
    import torch
    import token_dispatch_grouped_amd as moe
    from token_dispatch_grouped_amd.layer import MoeLayer
    w = WORKLOADS["microbatches_32k"]
    print(f"[fullsize] microbatches {w.microbatches} d={w.d} E={w.E} k={w.k} F={w.F}", flush=True)
    inp = make_inputs(w)
    W = inp["weights"]
    layer = MoeLayer(max(w.microbatches), w.d, w.E, w.k, w.F, moe.MOE_DTYPE_BF16)
    wgu = to_device(W["w_gu"], BF16)
    wdn = to_device(W["w_down"], BF16)
    dw_gu = torch.zeros(w.E, 2 * w.F, w.d, device="cuda")
    dw_dn = torch.zeros(w.E, w.d, w.F, device="cuda")
    tol = TOL[BF16]
    routes = []
    rng = np.random.default_rng(1)
    wgu64, wdn64 = to_f64(W["w_gu"], BF16), to_f64(W["w_down"], BF16)
    for i, mb in enumerate(inp["micro"]):
        T = mb["x"].shape[0]
        before = (dw_gu.clone(), dw_dn.clone())
        x = to_device(mb["x"], BF16)
        sv = layer.forward(T, x, wgu, wdn, logits=to_device(mb["logits"], F32))
        g = layer.backward(T, to_device(mb["dout"], BF16), wgu, wdn, dw_gu, dw_dn)
        torch.cuda.synchronize()
        r = oracle.route(mb["logits"].astype(np.float64), w.k)
        routes.append(r)
        if T == 0:
            assert torch.equal(before[0], dw_gu) and torch.equal(before[1], dw_dn)
            continue
        for key in ("topk_idx", "counts", "offsets", "row_of_slot", "src_of_row"):
            assert np.array_equal(getattr(sv, key).cpu().numpy(), r[key]), (i, key)
        toks = np.unique(np.concatenate([rng.integers(0, T, 16), [0, T - 1]]))
        out_s, sv_s = oracle.layer_fwd(to_f64(mb["x"], BF16)[toks], wgu64, wdn64, w.k,
                                       logits=mb["logits"][toks].astype(np.float64))
        g_s = oracle.layer_bwd(to_f64(mb["dout"], BF16)[toks], sv_s, wgu64, wdn64)
        assert_close(f"mb{i} out", to_host64(sv.out[toks.tolist()]), out_s, tol)
        assert_close(f"mb{i} dx", to_host64(g["dx"][toks.tolist()]), g_s["dx"], tol)
    del wgu64, wdn64
    # accumulated gradients of the heaviest and the lightest expert that is
    # live in every non-empty microbatch: the sum of the per-microbatch oracle
    # gradients
    nonempty = [(r, mb) for r, mb in zip(routes, inp["micro"]) if mb["x"].shape[0] > 0]
    live = [set(np.nonzero(r["counts"] > 0)[0].tolist()) for r, _ in nonempty]
    common = sorted(set.intersection(*live))
    total = {e: sum(int(r["counts"][e]) for r, _ in nonempty) for e in common}
    picks = sorted({max(common, key=lambda e: total[e]), min(common, key=lambda e: total[e])})
    for e in picks:
        acc_gu = 0.0
        acc_dn = 0.0
        for r, mb in nonempty:
            o = _expert_oracle(e, r, w.k, to_f64(mb["x"], BF16), to_f64(mb["dout"], BF16), W["w_gu"], W["w_down"])
            acc_gu = acc_gu + o["dw_gu"]
            acc_dn = acc_dn + o["dw_down"]
        print(f"[fullsize] accumulated dW check on expert {e} ({total[e]} rows over the microbatches)", flush=True)
        assert_close(f"dw_gu[{e}] accumulated", to_host64(dw_gu[e]), acc_gu, tol)
        assert_close(f"dw_down[{e}] accumulated", to_host64(dw_dn[e]), acc_dn, tol)
    # experts empty in every microbatch keep exactly zero gradients
    for ee in range(w.E):
        if all(int(r["counts"][ee]) == 0 for r in routes):
            assert float(dw_gu[ee].abs().max()) == 0.0 and float(dw_dn[ee].abs().max()) == 0.0


def test_fullsize_recompute_bitwise():
    """At the 32k EP-share size, the recomputing backward gives the same
    bits as the saved-activation path in every output and gradient (the
    latter is checked against the oracle above)."""
    import torch
    w = WORKLOADS["ep_share_32k"]
    print(f"[fullsize] recompute {w.name}: T={w.T} d={w.d} E={w.E} k={w.k} F={w.F}", flush=True)
    inp = make_inputs(w)
    lay_s, sv_s, g_s, dgu_s, ddn_s = _run_full(w, inp)
    res_s = {"out": sv_s.out.clone(), "y": sv_s.y.clone(), "dh": g_s["dh"].clone(),
             **{k: g_s[k].clone() for k in ("dy", "dtopk_w", "dlogits", "dx_perm", "dx")}}
    a_saved = sv_s.a.clone()
    del lay_s, sv_s, g_s
    torch.cuda.empty_cache()
    lay_r, sv_r, g_r, dgu_r, ddn_r = _run_full(w, inp, recompute=True)
    assert lay_r.h is None and lay_r.a is None
    for k, v in res_s.items():
        got = sv_r.out if k == "out" else sv_r.y if k == "y" else g_r[k]
        assert torch.equal(got, v), k
    assert torch.equal(dgu_r, dgu_s) and torch.equal(ddn_r, ddn_s)
    # the recomputed a sits after dH and the expert order in the backward workspace
    R, F = w.T * w.k, w.F
    align = lambda n: (n + 255) // 256 * 256
    off = align(R * 2 * F * 2) + align(w.E * 4)
    a_rc = lay_r.bwd_ws[off:off + R * F * 2].view(torch.bfloat16).view(R, F)
    assert torch.equal(a_rc, a_saved)
