"""Parity of the auxiliary losses and routing metrics (moe_aux_loss, through
the C ABI) with the fp64 oracle (oracle.aux), and of the router gradient
when the layer adds them (MOE_FLAG_ACCUMULATE_DLOGITS).

Bars (fp32 arithmetic): losses, every metric and dlogits within
max|gpu - ref| / max|ref| <= 1e-4 (per metric scalar, per per-expert array,
per dlogits tensor); the number of empty experts exact; results bitwise
identical run to run.
"""
import numpy as np
import pytest

import oracle
from tests.parity_util import TOL, assert_close, to_device, to_host64
from workloads import BF16, F32, WORKLOADS, make_inputs, small_workload, to_f64

pytestmark = pytest.mark.gpu
TOL_F32 = TOL[F32]


def _gpu_aux(logits, E, k, alpha, beta, dlogits_init=None):
    """Route the given fp32 logits on the GPU, then run moe_aux_loss."""
    import torch
    import token_dispatch_grouped_amd as m
    T = logits.shape[0]
    s = m.make_shape(T, 64, E, k, 64, m.MOE_DTYPE_BF16, 0)
    rws, _, _ = m.moe_workspace_size(s)
    ws = torch.empty(max(rws, 256), dtype=torch.uint8, device="cuda")
    lg = to_device(np.ascontiguousarray(logits, dtype=np.float32), F32)
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    tw = torch.empty(T, k, dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    ros = torch.empty(T, k, dtype=torch.int32, device="cuda")
    sor = torch.empty(T * k, dtype=torch.int32, device="cuda")
    m.moe_route(s, None, None, None, lg, idx, tw, counts, offs, ros, sor, ws, ws.numel())
    losses = torch.full((2,), float("nan"), device="cuda")
    metrics = torch.full((m.MOE_METRIC_SCALARS + 2 * E,), float("nan"), device="cuda")
    acc = dlogits_init is not None
    dl = (to_device(np.ascontiguousarray(dlogits_init, dtype=np.float32), F32) if acc
          else torch.full((T, E), float("nan"), device="cuda"))
    m.moe_aux_loss(s, lg, counts, m.make_aux_config(alpha, beta, acc), losses, metrics, dl, ws, ws.numel())
    torch.cuda.synchronize()
    return counts.cpu().numpy(), to_host64(losses), to_host64(metrics), to_host64(dl)


def _check(logits, counts_gpu, k, alpha, beta, losses, metrics, dl, dl_init=None):
    T, E = logits.shape
    lg64 = logits.astype(np.float32).astype(np.float64)
    r = oracle.route(lg64, k)
    assert np.array_equal(counts_gpu, r["counts"]), "counts"
    lb, lz = oracle.aux_losses(lg64, r["counts"], k)
    assert_close("L_bal", losses[0:1], np.array([lb]), TOL_F32)
    assert_close("L_z", losses[1:2], np.array([lz]), TOL_F32)
    met = oracle.routing_metrics(lg64, r["counts"], k)
    for i, name in enumerate(oracle.METRIC_NAMES):
        if name == "empty_experts":
            assert metrics[i] == met[i], name
        else:
            assert_close(name, metrics[i:i + 1], met[i:i + 1], TOL_F32)
    assert_close("f_e", metrics[5:5 + E], met[5:5 + E], TOL_F32)
    assert_close("P_e", metrics[5 + E:], met[5 + E:], TOL_F32)
    want = oracle.aux_losses_grad(lg64, r["counts"], k, alpha, beta)
    if dl_init is not None:
        want = want + dl_init.astype(np.float32).astype(np.float64)
    assert_close("dlogits", dl, want, TOL_F32)


CASES = [
    # T, E, k, routing, n_empty, seed
    (1, 4, 2, "normal", 0, 61),
    (255, 8, 2, "normal", 0, 62),
    (256, 32, 8, "zipf", 2, 63),
    (257, 64, 8, "zipf", 5, 64),
    (1000, 256, 16, "normal", 0, 65),
    (3000, 1, 1, "normal", 0, 66),
    (4099, 16, 4, "zipf", 3, 67),
    # every split of a row over lanes (1, 4 or 8 lanes; 8, 16 or 32 values per lane; rows of single values when E is
    # not a multiple of 4) and, past 65536 tokens, workgroups that take more than one pass over their tokens
    (333, 100, 3, "zipf", 4, 72),
    (129, 129, 5, "normal", 0, 73),
    (700, 31, 4, "zipf", 2, 74),
    (130, 5, 2, "normal", 0, 75),
    (70000, 64, 8, "zipf", 3, 76),
]


@pytest.mark.parametrize("T,E,k,routing,n_empty,seed", CASES)
def test_aux_small(T, E, k, routing, n_empty, seed):
    print(f"[aux] T={T} E={E} k={k} {routing} empty={n_empty}", flush=True)
    w = small_workload(T, 64, E, k, 64, BF16, routing, seed=seed, n_empty=n_empty)
    lg = make_inputs(w)["micro"][0]["logits"]
    c, losses, met, dl = _gpu_aux(lg, E, k, 0.01, 1e-3)
    _check(lg, c, k, 0.01, 1e-3, losses, met, dl)


def test_aux_minus_infinity_and_accumulate():
    w = small_workload(700, 64, 16, 4, 64, BF16, "normal", seed=68)
    lg = make_inputs(w)["micro"][0]["logits"].copy()
    lg[::3, 2] = -np.inf
    lg[1::7, 9] = -np.inf
    init = np.random.default_rng(69).normal(0, 1e-3, lg.shape).astype(np.float32)
    c, losses, met, dl = _gpu_aux(lg, 16, 4, 0.05, 0.01, dlogits_init=init)
    _check(lg, c, 4, 0.05, 0.01, losses, met, dl, dl_init=init)


@pytest.mark.parametrize("name", ["ep_share_32k", "large_share_zipf", "large_share_uniform"])
def test_aux_fullsize_and_deterministic(name):
    w = WORKLOADS[name]
    print(f"[aux] full size {name}: T={w.T} E={w.E} k={w.k}", flush=True)
    lg = make_inputs(w)["micro"][0]["logits"]
    c, losses, met, dl = _gpu_aux(lg, w.E, w.k, 0.01, 1e-3)
    _check(lg, c, w.k, 0.01, 1e-3, losses, met, dl)
    c2, losses2, met2, dl2 = _gpu_aux(lg, w.E, w.k, 0.01, 1e-3)
    assert np.array_equal(losses, losses2) and np.array_equal(met, met2) and np.array_equal(dl, dl2)


def test_layer_router_with_aux_losses():
    """Router mode: the aux gradient joins dlogits before the routing-weight
    gradient, and dx_router / dw_router back-propagate the sum."""
    import torch
    import token_dispatch_grouped_amd as m
    from token_dispatch_grouped_amd.layer import MoeLayer
    w = small_workload(512, 256, 8, 2, 256, BF16, "router", seed=70, n_empty=1)
    inp = make_inputs(w)
    W, mb = inp["weights"], inp["micro"][0]
    alpha, beta = 0.02, 1e-3
    layer = MoeLayer(512, w.d, w.E, w.k, w.F, m.MOE_DTYPE_BF16, router=True, aux=(alpha, beta))
    x = to_device(mb["x"], BF16)
    wgu, wdn, wr = to_device(W["w_gu"], BF16), to_device(W["w_down"], BF16), to_device(W["w_router"], BF16)
    bias = to_device(W["bias"], F32)
    dgu = torch.zeros(w.E, 2 * w.F, w.d, device="cuda")
    ddn = torch.zeros(w.E, w.d, w.F, device="cuda")
    dwr = torch.zeros(w.E, w.d, device="cuda")
    sv = layer.forward(512, x, wgu, wdn, w_router=wr, bias=bias)
    g = layer.backward(512, to_device(mb["dout"], BF16), wgu, wdn, dgu, ddn, x=x, w_router=wr, dw_router=dwr)
    torch.cuda.synchronize()
    lg_gpu = to_host64(sv.logits)        # routing is checked on the GPU's own fp32 logits (see test_gpu_parity)
    counts = sv.counts.cpu().numpy()
    x64, wr64 = to_f64(mb["x"], BF16), to_f64(W["w_router"], BF16)
    wgu64, wdn64 = to_f64(W["w_gu"], BF16), to_f64(W["w_down"], BF16)
    out, svo = oracle.layer_fwd(x64, wgu64, wdn64, w.k, logits=lg_gpu)
    go = oracle.layer_bwd(to_f64(mb["dout"], BF16), svo, wgu64, wdn64)
    aux_grad = oracle.aux_losses_grad(lg_gpu, counts, w.k, alpha, beta)
    total = go["dlogits"] + aux_grad
    dxr, dwr_ref = oracle.router_bwd(total, x64, wr64)
    lb, lz = oracle.aux_losses(lg_gpu, counts, w.k)
    assert_close("L_bal", to_host64(layer.aux_losses[0:1]), np.array([lb]), TOL_F32)
    assert_close("L_z", to_host64(layer.aux_losses[1:2]), np.array([lz]), TOL_F32)
    assert_close("metrics", to_host64(layer.metrics), oracle.routing_metrics(lg_gpu, counts, w.k), TOL_F32)
    tol = TOL[BF16]
    assert_close("dlogits (routing + aux)", to_host64(g["dlogits"]), total, tol)
    assert_close("dx_router", to_host64(g["dx_router"]), dxr, tol)
    assert_close("dw_router", to_host64(dwr), dwr_ref, tol)
    assert_close("dx", to_host64(g["dx"]), go["dx"] + dxr, tol)


@pytest.mark.parametrize("renorm", [False, True])
def test_layer_logits_with_aux_losses(renorm):
    """Given-logits mode (the 32k workloads' mode) with the auxiliary losses:
    dlogits = routing-weight gradient (plain or renormalised) + aux gradient,
    summed by moe_route_bwd under MOE_FLAG_ACCUMULATE_DLOGITS."""
    import torch
    import token_dispatch_grouped_amd as m
    from token_dispatch_grouped_amd.layer import MoeLayer
    w = small_workload(777, 128, 16, 4, 128, BF16, "zipf", seed=71, n_empty=2)
    inp = make_inputs(w)
    W, mb = inp["weights"], inp["micro"][0]
    alpha, beta = 0.05, 2e-3
    layer = MoeLayer(777, w.d, w.E, w.k, w.F, m.MOE_DTYPE_BF16, renorm=renorm, aux=(alpha, beta))
    wgu, wdn = to_device(W["w_gu"], BF16), to_device(W["w_down"], BF16)
    dgu = torch.zeros(w.E, 2 * w.F, w.d, device="cuda")
    ddn = torch.zeros(w.E, w.d, w.F, device="cuda")
    layer.forward(777, to_device(mb["x"], BF16), wgu, wdn, logits=to_device(mb["logits"], F32))
    g = layer.backward(777, to_device(mb["dout"], BF16), wgu, wdn, dgu, ddn)
    torch.cuda.synchronize()
    lg = mb["logits"].astype(np.float64)
    wgu64, wdn64 = to_f64(W["w_gu"], BF16), to_f64(W["w_down"], BF16)
    _, svo = oracle.layer_fwd(to_f64(mb["x"], BF16), wgu64, wdn64, w.k, logits=lg, renorm=renorm)
    go = oracle.layer_bwd(to_f64(mb["dout"], BF16), svo, wgu64, wdn64, renorm=renorm)
    total = go["dlogits"] + oracle.aux_losses_grad(lg, svo["counts"], w.k, alpha, beta)
    assert_close("dlogits (routing + aux)", to_host64(g["dlogits"]), total, TOL[BF16])
    assert_close("dx", to_host64(g["dx"]), go["dx"], TOL[BF16])
    lb, lz = oracle.aux_losses(lg, svo["counts"], w.k)
    assert_close("L_bal", to_host64(layer.aux_losses[0:1]), np.array([lb]), TOL_F32)
    assert_close("L_z", to_host64(layer.aux_losses[1:2]), np.array([lz]), TOL_F32)


def test_empty_microbatch_writes_zero_losses():
    """T = 0 (the empty-work case): losses and metrics of the previous call
    are overwritten with the empty microbatch's values (losses 0, every
    metric 0 but empty_experts = E), so a caller summing per-microbatch
    losses adds nothing for it; NULL logits, counts and dlogits are accepted."""
    import torch
    import token_dispatch_grouped_amd as m
    E, k = 12, 3
    s = m.make_shape(0, 64, E, k, 64, m.MOE_DTYPE_BF16, 0)
    losses = torch.full((2,), 5.0, device="cuda")
    metrics = torch.full((m.MOE_METRIC_SCALARS + 2 * E,), 5.0, device="cuda")
    m.moe_aux_loss(s, None, None, m.make_aux_config(0.01, 0.001), losses, metrics, None, None, 0)
    torch.cuda.synchronize()
    want = oracle.routing_metrics(np.zeros((0, E)), np.zeros(E, np.int32), k)
    assert to_host64(losses).tolist() == list(oracle.aux_losses(np.zeros((0, E)), np.zeros(E, np.int32), k))
    assert np.array_equal(to_host64(metrics), want)
