"""Parity at full workload sizes, in the launch configuration the bench times.

At T=32768 the fp64 oracle cannot run the whole layer in seconds, so:
  * routing and dispatch tables are compared in full, bit for bit (the
    oracle's selection is cheap);
  * the dispatched copy is compared bit for bit on sampled rows;
  * forward outputs and the token-side gradients are compared on sampled
    tokens: the layer is per-token, so the oracle run on the sub-batch of
    sampled tokens gives exactly those tokens' results;
  * weight gradients are compared in full for the smallest non-empty
    expert (the oracle runs that expert's FFN on its own rows), and empty
    experts must have exactly zero gradient.
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


@pytest.mark.parametrize("name", ["ep_share_32k", "large_share_zipf", "large_share_uniform"])
def test_fullsize_sampled(name):
    w = WORKLOADS[name]
    print(f"[fullsize] {name}: T={w.T} d={w.d} E={w.E} k={w.k} F={w.F}", flush=True)
    inp = make_inputs(w)
    mb = inp["micro"][0]
    W = inp["weights"]
    T, k = w.T, w.k
    layer, sv, g, dw_gu, dw_dn = _run_full(w, inp)
    tol = TOL[BF16]

    # --- routing and dispatch tables: whole tensors, bit-exact
    r = oracle.route(mb["logits"].astype(np.float64), k)
    for key in ("topk_idx", "counts", "offsets", "row_of_slot", "src_of_row"):
        assert np.array_equal(getattr(sv, key).cpu().numpy(), r[key]), key
    assert_close("topk_w", to_host64(sv.topk_w), r["topk_w"], TOL_ROUTING)
    counts = r["counts"]
    assert (counts == 0).sum() == w.n_empty

    # --- dispatched copy on sampled rows, bit-exact
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.integers(0, T * k, 4000), [0, T * k - 1]]))
    xp = to_host64(sv.x_perm[rows.tolist()])
    want = to_f64(mb["x"], BF16)[r["src_of_row"][rows] // k]
    assert np.array_equal(xp, want), "x_perm rows"

    # --- sampled tokens: forward outputs and token-side gradients
    toks = np.unique(np.concatenate([rng.integers(0, T, 40), [0, T - 1]]))
    wgu64, wdn64 = to_f64(W["w_gu"], BF16), to_f64(W["w_down"], BF16)
    xs = to_f64(mb["x"], BF16)[toks]
    ds = to_f64(mb["dout"], BF16)[toks]
    out_s, sv_s = oracle.layer_fwd(xs, wgu64, wdn64, k, logits=mb["logits"][toks].astype(np.float64))
    g_s = oracle.layer_bwd(ds, sv_s, wgu64, wdn64)
    assert_close("out", to_host64(sv.out[toks.tolist()]), out_s, tol)
    assert_close("dx", to_host64(g["dx"][toks.tolist()]), g_s["dx"], tol)
    assert_close("dtopk_w", to_host64(g["dtopk_w"][toks.tolist()]), g_s["dtopk_w"], tol)
    assert_close("dlogits", to_host64(g["dlogits"][toks.tolist()]), g_s["dlogits"], tol)
    # per-slot saved tensors: map the sub-batch's rows to the full batch's rows
    full_rows = r["row_of_slot"][toks].reshape(-1)
    sub_rows = sv_s["row_of_slot"].reshape(-1)
    for key, gpu_t in (("h", sv.h), ("a", sv.a), ("y", sv.y), ("dy", g["dy"]), ("dx_perm", g["dx_perm"]),
                       ("dh", g["dh"])):
        ref = (sv_s if key in ("h", "a", "y") else g_s)[key][sub_rows]
        assert_close(key, to_host64(gpu_t[full_rows.tolist()]), ref, tol)

    # --- weight gradients: the smallest non-empty expert in full
    e = int(np.argmin(np.where(counts > 0, counts, np.iinfo(np.int32).max)))
    lo, hi = int(r["offsets"][e]), int(r["offsets"][e + 1])
    slots = r["src_of_row"][lo:hi]
    t_of = slots // k
    x_e = to_f64(mb["x"], BF16)[t_of]
    w_e = r["topk_w"].reshape(-1)[slots][:, None]
    dout_e = to_f64(mb["dout"], BF16)[t_of]
    off1 = np.array([0, hi - lo], dtype=np.int32)
    h_e, a_e, y_e = oracle.expert_ffn_fwd(x_e, wgu64[e:e + 1], wdn64[e:e + 1], off1)
    dy_e, _ = oracle.unpermute_combine_bwd(dout_e, y_e, w_e, np.arange(hi - lo, dtype=np.int32)[:, None])
    _, dwgu_e, dwdn_e, _ = oracle.expert_ffn_bwd(dy_e, x_e, h_e, a_e, wgu64[e:e + 1], wdn64[e:e + 1], off1)
    print(f"[fullsize] dW check on expert {e} with {hi - lo} rows", flush=True)
    assert_close(f"dw_gu[{e}]", to_host64(dw_gu[e]), dwgu_e[0], tol)
    assert_close(f"dw_down[{e}]", to_host64(dw_dn[e]), dwdn_e[0], tol)
    for ee in np.nonzero(counts == 0)[0]:
        assert float(dw_gu[int(ee)].abs().max()) == 0.0 and float(dw_dn[int(ee)].abs().max()) == 0.0
    # every output finite
    import torch
    for t in (sv.out, sv.y, sv.h, g["dx"], g["dx_perm"], dw_gu, dw_dn):
        assert bool(torch.isfinite(t).all())


def _expert_dw_oracle(w, mb, W, r, e):
    """fp64 weight gradients of expert e from one microbatch, computed by the
    oracle on that expert's own rows."""
    k = w.k
    lo, hi = int(r["offsets"][e]), int(r["offsets"][e + 1])
    wgu64, wdn64 = to_f64(W["w_gu"][e:e + 1], BF16), to_f64(W["w_down"][e:e + 1], BF16)
    if hi == lo:
        return np.zeros(wgu64.shape[1:]), np.zeros(wdn64.shape[1:])
    slots = r["src_of_row"][lo:hi]
    t_of = slots // k
    x_e = to_f64(mb["x"], BF16)[t_of]
    w_e = r["topk_w"].reshape(-1)[slots][:, None]
    dout_e = to_f64(mb["dout"], BF16)[t_of]
    off1 = np.array([0, hi - lo], dtype=np.int32)
    h_e, a_e, y_e = oracle.expert_ffn_fwd(x_e, wgu64, wdn64, off1)
    dy_e, _ = oracle.unpermute_combine_bwd(dout_e, y_e, w_e, np.arange(hi - lo, dtype=np.int32)[:, None])
    _, dwgu, dwdn, _ = oracle.expert_ffn_bwd(dy_e, x_e, h_e, a_e, wgu64, wdn64, off1)
    return dwgu[0], dwdn[0]


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
        wgu64, wdn64 = to_f64(W["w_gu"], BF16), to_f64(W["w_down"], BF16)
        out_s, sv_s = oracle.layer_fwd(to_f64(mb["x"], BF16)[toks], wgu64, wdn64, w.k,
                                       logits=mb["logits"][toks].astype(np.float64))
        g_s = oracle.layer_bwd(to_f64(mb["dout"], BF16)[toks], sv_s, wgu64, wdn64)
        assert_close(f"mb{i} out", to_host64(sv.out[toks.tolist()]), out_s, tol)
        assert_close(f"mb{i} dx", to_host64(g["dx"][toks.tolist()]), g_s["dx"], tol)
    # accumulated gradients of one expert that is non-empty in every non-empty
    # microbatch: the sum of the per-microbatch oracle gradients
    live = [np.nonzero(r["counts"] > 0)[0] for r, mb in zip(routes, inp["micro"]) if mb["x"].shape[0] > 0]
    common = sorted(set(live[0]).intersection(*map(set, live[1:])))
    e = min(common, key=lambda ee: sum(int(r["counts"][ee]) for r in routes))
    acc_gu = 0.0
    acc_dn = 0.0
    for r, mb in zip(routes, inp["micro"]):
        if mb["x"].shape[0] == 0:
            continue
        a, b = _expert_dw_oracle(w, mb, W, r, e)
        acc_gu = acc_gu + a
        acc_dn = acc_dn + b
    print(f"[fullsize] accumulated dW check on expert {e}", flush=True)
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
