"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Inputs are the seeded synthetic workloads; the oracle never sees anything
the GPU produced except where stated (routing tables of a router run are
checked by feeding the GPU's fp32 logits to the oracle's selection, since
the router GEMM's rounding may legitimately differ from fp64).

Bars: integer tables and the dispatched copy bit-exact; floats within
max|gpu-ref|/max|ref| <= 2e-2 (bf16 layer) or 1e-4 (fp32 layer); routing
weights (pure fp32 arithmetic) within 1e-4.
"""
import numpy as np
import pytest

import oracle
from tests.parity_util import TOL, TOL_ROUTING, assert_close, to_device, to_host64
from workloads import BF16, F32, WORKLOADS, make_inputs, small_workload, tie_logits, to_f64

pytestmark = pytest.mark.gpu


def _moe():
    import token_dispatch_grouped_amd as m
    from token_dispatch_grouped_amd.layer import MoeLayer
    return m, MoeLayer


def gpu_run(w, inp, renorm=False, logits_override=None, sentinel=False, recompute=False):
    """Run every microbatch forward+backward on the GPU; dW accumulate.
    With recompute, h is not kept (None in the results) and a is read from
    the forward workspace right after the forward."""
    import torch
    m, MoeLayer = _moe()
    dt = m.MOE_DTYPE_BF16 if w.dtype == BF16 else m.MOE_DTYPE_F32
    router = w.routing == "router"
    Tmax = max(max(w.microbatches), 1)
    layer = MoeLayer(Tmax, w.d, w.E, w.k, w.F, dt, renorm=renorm, router=router, recompute=recompute)
    if sentinel:
        for name in ("x_perm", "h", "a", "y", "out", "dy", "dx_perm", "dx", "logits", "topk_w", "dtopk_w",
                     "dlogits"):
            getattr(layer, name).fill_(float("nan"))
        for name in ("topk_idx", "row_of_slot", "src_of_row", "counts", "offsets"):
            getattr(layer, name).fill_(-7)
    W = inp["weights"]
    wgu = to_device(W["w_gu"], w.dtype)
    wdn = to_device(W["w_down"], w.dtype)
    wr = to_device(W["w_router"], w.dtype) if router else None
    bias = to_device(W["bias"], F32) if router else None
    dw_gu = torch.zeros(w.E, 2 * w.F, w.d, dtype=torch.float32, device="cuda")
    dw_down = torch.zeros(w.E, w.d, w.F, dtype=torch.float32, device="cuda")
    dw_router = torch.zeros(w.E, w.d, dtype=torch.float32, device="cuda") if router else None
    res = []
    for i, mb in enumerate(inp["micro"]):
        T = mb["x"].shape[0]
        x = to_device(mb["x"], w.dtype)
        dout = to_device(mb["dout"], w.dtype)
        lg = None
        if not router:
            lg = logits_override[i] if logits_override is not None else mb["logits"]
            lg = to_device(np.ascontiguousarray(lg, dtype=np.float32), F32)
        before = (dw_gu.clone(), dw_down.clone())
        sv = layer.forward(T, x, wgu, wdn, logits=lg, w_router=wr, bias=bias)
        a_fwd = to_host64(layer.fwd_a_view(T)) if recompute else None
        g = layer.backward(T, dout, wgu, wdn, dw_gu, dw_down, x=x, w_router=wr, dw_router=dw_router)
        torch.cuda.synchronize()
        r = {k: to_host64(getattr(sv, k)) for k in ("logits", "topk_w", "x_perm", "y", "out")}
        r["h"] = None if recompute else to_host64(sv.h)
        r["a"] = a_fwd if recompute else to_host64(sv.a)
        for k in ("topk_idx", "row_of_slot", "src_of_row", "counts", "offsets"):
            r[k] = getattr(sv, k).cpu().numpy()
        for k in ("dy", "dtopk_w", "dlogits", "dx_perm", "dx", "dh"):
            r[k] = to_host64(g[k])
        if router:
            r["dx_router"] = to_host64(g["dx_router"])
        r["dw_unchanged"] = bool(torch.equal(before[0], dw_gu) and torch.equal(before[1], dw_down))
        res.append(r)
    acc = {"dw_gu": to_host64(dw_gu), "dw_down": to_host64(dw_down)}
    if router:
        acc["dw_router"] = to_host64(dw_router)
    return res, acc


def oracle_run(w, inp, renorm=False, logits_override=None):
    W = inp["weights"]
    wgu = to_f64(W["w_gu"], w.dtype)
    wdn = to_f64(W["w_down"], w.dtype)
    router = w.routing == "router"
    wr = to_f64(W["w_router"], w.dtype) if router else None
    bias = W["bias"].astype(np.float64) if router else None
    acc = {"dw_gu": np.zeros_like(wgu), "dw_down": np.zeros_like(wdn)}
    if router:
        acc["dw_router"] = np.zeros_like(wr)
    res = []
    for i, mb in enumerate(inp["micro"]):
        x = to_f64(mb["x"], w.dtype)
        dout = to_f64(mb["dout"], w.dtype)
        if router:
            out, sv = oracle.layer_fwd(x, wgu, wdn, w.k, w_router=wr, bias=bias, renorm=renorm)
        else:
            lg = logits_override[i] if logits_override is not None else mb["logits"]
            out, sv = oracle.layer_fwd(x, wgu, wdn, w.k, logits=lg.astype(np.float64), renorm=renorm)
        g = oracle.layer_bwd(dout, sv, wgu, wdn, x=x, w_router=wr, renorm=renorm)
        acc["dw_gu"] += g["dw_gu"]
        acc["dw_down"] += g["dw_down"]
        if router:
            acc["dw_router"] += g["dw_router"]
        r = dict(sv)
        r["out"] = out
        r.update(g)
        res.append(r)
    return res, acc


def compare(w, gres, gacc, ores, oacc, renorm=False):
    tol = TOL[w.dtype]
    errs = {}
    for i, (g, o) in enumerate(zip(gres, ores)):
        T = o["out"].shape[0]
        if w.routing == "router" and T:
            errs["logits"] = assert_close("logits", g["logits"], o["logits"], tol)
            # selection from the GPU's own fp32 logits must match exactly
            r2 = oracle.route(g["logits"], w.k, renorm)
            for k in ("topk_idx", "counts", "offsets", "row_of_slot", "src_of_row"):
                assert np.array_equal(g[k], r2[k]), f"mb{i} {k} (oracle selection on GPU logits)"
            assert np.array_equal(r2["topk_idx"], o["topk_idx"]), \
                f"mb{i}: routing flipped between fp64 and GPU fp32 logits"
        if T == 0:
            assert g["dw_unchanged"], "empty microbatch changed dW"
            continue
        for k in ("topk_idx", "counts", "offsets", "row_of_slot", "src_of_row"):
            assert np.array_equal(g[k], o[k]), f"mb{i} {k} not bit-exact"
        assert np.array_equal(g["x_perm"], o["x_perm"]), f"mb{i} x_perm not bit-exact"
        errs["topk_w"] = assert_close("topk_w", g["topk_w"], o["topk_w"], TOL_ROUTING if w.routing != "router"
                                      else tol)
        for k in ("h", "a", "y", "out", "dy", "dtopk_w", "dlogits", "dx_perm", "dh", "dx"):
            if g[k] is None:  # h is not kept under recompute
                continue
            errs[k] = assert_close(f"mb{i} {k}", g[k], o[k], tol)
        if w.routing == "router":
            errs["dx_router"] = assert_close(f"mb{i} dx_router", g["dx_router"], o["dx_router"], tol)
    for k in oacc:
        errs[k] = assert_close(k, gacc[k], oacc[k], tol)
    # per-expert slices of dW: empty experts exactly zero, others within the bar
    for k in ("dw_gu", "dw_down"):
        for e in range(w.E):
            if np.max(np.abs(oacc[k][e])) == 0.0:
                assert np.all(gacc[k][e] == 0.0), f"{k}[{e}] of an empty expert is not exactly zero"
            else:
                assert_close(f"{k}[{e}]", gacc[k][e], oacc[k][e], tol)
    return errs


SMALL_CASES = [
    # name, workload, renorm
    ("tiny_f32_router", WORKLOADS["tiny_f32"], False),
    ("tiny_f32_router_renorm", WORKLOADS["tiny_f32"], True),
    ("bf16_ragged_tiles_zipf", small_workload(600, 256, 8, 2, 192, BF16, "zipf", seed=21, n_empty=2), False),
    ("bf16_k_equals_E", small_workload(333, 128, 4, 4, 64, BF16, "normal", seed=22), False),
    ("bf16_single_expert", small_workload(1, 64, 1, 1, 64, BF16, "normal", seed=23), False),
    ("bf16_E1_k1_many", small_workload(300, 128, 1, 1, 128, BF16, "normal", seed=24), False),
    ("bf16_renorm_k8", small_workload(257, 128, 32, 8, 128, BF16, "zipf", seed=25, n_empty=3), True),
    ("bf16_router_small", small_workload(512, 256, 8, 2, 256, BF16, "router", seed=26, n_empty=1), False),
    ("f32_zipf", small_workload(200, 128, 16, 4, 128, F32, "zipf", seed=27, n_empty=4), False),
    ("bf16_E256_k16", small_workload(130, 64, 256, 16, 64, BF16, "normal", seed=28), False),
    # F = 64: the down forward is one 64-deep stage, and with d = 2048 its ~560 tiles give every persistent
    # workgroup several, so a tile whose only stage was issued during the previous tile's epilogue runs
    ("bf16_F64_multi_tile", small_workload(4096, 2048, 8, 4, 64, BF16, "zipf", seed=29, n_empty=1), False),
    # every ragged-M product with more tiles than workgroups (gate/up forward ~2.6 per workgroup, the others
    # 1.3-1.7) and Zipf tails of every length, so the next tile's first stage is issued from each epilogue
    # (plain store, SwiGLU forward after h, SwiGLU backward in a last band held in either buffer) and the
    # whole result is compared, not a sample
    ("bf16_persistent_all_epilogues", small_workload(6144, 1024, 16, 4, 768, BF16, "zipf", seed=30, n_empty=2),
     False),
    # rows wider than one pass of the combine backward (2048 16-byte chunks per wavefront): d = 16448 in bf16
    # and d = 8256 in fp32 take a second pass over the row's last chunks
    ("bf16_wide_d16448", small_workload(6, 16448, 4, 2, 64, BF16, "normal", seed=39), False),
    ("f32_wide_d8256", small_workload(5, 8256, 3, 2, 64, F32, "normal", seed=40), False),
    # the combine backward's three forms at their edges: one workgroup per token with a ragged second pass
    # (264 and 272 chunks), one workgroup per (token, slot) row with a ragged second chunk loop (520 chunks),
    # k = 3 and T = 13 so logical rows past the last token end the loop, and the per-row form in fp32
    ("bf16_d2112_cbwd_token_tail", small_workload(9, 2112, 4, 2, 64, BF16, "normal", seed=41), False),
    ("f32_d1088_cbwd_token_tail", small_workload(7, 1088, 3, 2, 64, F32, "normal", seed=42), False),
    ("bf16_d4160_cbwd_row_tail", small_workload(13, 4160, 5, 3, 64, BF16, "normal", seed=43), False),
    ("f32_d2048_cbwd_row", small_workload(11, 2048, 4, 1, 64, F32, "zipf", seed=44), False),
    # the down weight gradient's edge tiles (F an odd multiple of 128, d a multiple of 512: the last 128 columns
    # of dW_down as 512 x 128 tiles): beside 256 x 256 tiles with empty experts, and alone (F = 128, no 256-wide
    # column tile at all)
    ("bf16_wgrad_edge_tiles", small_workload(900, 1024, 8, 2, 384, BF16, "zipf", seed=45, n_empty=2), False),
    ("bf16_wgrad_edge_only", small_workload(333, 512, 5, 3, 128, BF16, "normal", seed=46), False),
    # F an odd multiple of 128 with experts of many row tiles: the down dgrad's half-empty last column tile
    # (columns past F clamped on load, never stored) on Zipf experts of 11, 6 and 8 row tiles and an empty
    # one, beside full 256 x 256 tiles, in every product
    ("bf16_F640_half_column_tiles", small_workload(3000, 256, 4, 2, 640, BF16, "zipf", seed=47, n_empty=1), False),
]


def _random_cases(n=14, seed=2024):
    """Seeded random layer shapes within the supported matrix (d, F multiples of 64, k <= E <= 256),
    sized so the oracle finishes in a second or two: tile edges, ragged tails, empty experts and both
    dtypes in combinations the hand-picked cases do not cover."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dtype = BF16 if rng.random() < 0.75 else F32
        E = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 31, 64, 100]))
        k = int(rng.integers(1, min(E, 8) + 1))
        d = 64 * int(rng.integers(1, 9))
        F = 64 * int(rng.integers(1, 9))
        T = int(rng.integers(1, 2049))
        if 18.0 * T * k * d * F > 3e10:
            continue
        routing = "zipf" if rng.random() < 0.6 else "normal"
        n_empty = int(rng.integers(0, E - k + 1)) if routing == "zipf" and E > k else 0
        renorm = bool(rng.random() < 0.3)
        s = int(rng.integers(100, 10_000))
        name = f"rand{len(cases)}_T{T}_d{d}_E{E}_k{k}_F{F}_{dtype}_{routing}{n_empty}{'_renorm' if renorm else ''}"
        cases.append((name, small_workload(T, d, E, k, F, dtype, routing, seed=s, n_empty=n_empty), renorm))
    return cases


RANDOM_CASES = _random_cases()


def _random_wide_cases(n=30, seed=777):
    """Seeded random shapes over a wider part of the matrix than _random_cases: T from 0 to 4096, d and F up to
    1024, E up to 256 (odd counts among them), k up to 16, both dtypes, renorm, Zipf tails with empty experts;
    each case's oracle work is bounded (18*T*k*d*F <= 4e10 FLOP)."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dtype = BF16 if rng.random() < 0.8 else F32
        E = int(rng.choice([1, 2, 3, 4, 7, 8, 16, 32, 33, 64, 100, 128, 255, 256]))
        k = int(rng.integers(1, min(E, 16) + 1))
        d = 64 * int(rng.integers(1, 17))
        F = 64 * int(rng.integers(1, 17))
        T = int(rng.integers(0, 4097))
        if 18.0 * max(T, 1) * k * d * F > 4e10:
            continue
        routing = "zipf" if rng.random() < 0.6 else "normal"
        n_empty = int(rng.integers(0, E - k + 1)) if routing == "zipf" and E > k else 0
        renorm = bool(rng.random() < 0.3)
        s = int(rng.integers(100, 100000))
        name = f"wide{len(cases)}_T{T}_d{d}_E{E}_k{k}_F{F}_{dtype}_{routing}{n_empty}{'_renorm' if renorm else ''}"
        cases.append((name, small_workload(T, d, E, k, F, dtype, routing, seed=s, n_empty=n_empty), renorm))
    return cases


RANDOM_WIDE_CASES = _random_wide_cases()


@pytest.mark.parametrize("name,w,renorm", RANDOM_CASES, ids=[c[0] for c in RANDOM_CASES])
def test_layer_random_shapes(name, w, renorm):
    print(f"[parity] {name}", flush=True)
    inp = make_inputs(w)
    gres, gacc = gpu_run(w, inp, renorm)
    ores, oacc = oracle_run(w, inp, renorm)
    compare(w, gres, gacc, ores, oacc, renorm)


@pytest.mark.parametrize("name,w,renorm", RANDOM_WIDE_CASES, ids=[c[0] for c in RANDOM_WIDE_CASES])
def test_layer_random_wide_shapes(name, w, renorm):
    print(f"[parity] {name}", flush=True)
    inp = make_inputs(w)
    gres, gacc = gpu_run(w, inp, renorm)
    ores, oacc = oracle_run(w, inp, renorm)
    compare(w, gres, gacc, ores, oacc, renorm)


@pytest.mark.parametrize("name,w,renorm", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_layer_small(name, w, renorm):
    print(f"[parity] {name} T={w.T} d={w.d} E={w.E} k={w.k} F={w.F} {w.dtype}", flush=True)
    inp = make_inputs(w)
    gres, gacc = gpu_run(w, inp, renorm)
    ores, oacc = oracle_run(w, inp, renorm)
    compare(w, gres, gacc, ores, oacc, renorm)


def test_all_tokens_one_expert():
    w = small_workload(700, 128, 8, 1, 128, BF16, "normal", seed=31)
    inp = make_inputs(w)
    lg = inp["micro"][0]["logits"].copy()
    lg[:, 5] = 50.0
    gres, gacc = gpu_run(w, inp, logits_override=[lg])
    ores, oacc = oracle_run(w, inp, logits_override=[lg])
    assert gres[0]["counts"].tolist() == [0] * 5 + [700] + [0] * 2
    compare(w, gres, gacc, ores, oacc)


def test_tie_breaking_lowest_id():
    w = small_workload(1000, 64, 16, 4, 64, BF16, "normal", seed=32)
    inp = make_inputs(w)
    lg = [tie_logits(1000, 16, 5, levels=2)]
    gres, gacc = gpu_run(w, inp, logits_override=lg)
    ores, oacc = oracle_run(w, inp, logits_override=lg)
    compare(w, gres, gacc, ores, oacc)


def test_nonfinite_logits():
    """-inf never beats a finite logit; NaN ranks below -inf; -0.0 ties +0.0."""
    w = small_workload(64, 64, 8, 4, 64, BF16, "normal", seed=33)
    inp = make_inputs(w)
    lg = inp["micro"][0]["logits"].copy()
    lg[::3, 2] = -np.inf
    lg[1::5, 6] = np.nan
    lg[2::4, 0] = -0.0
    lg[2::4, 1] = 0.0
    gres, _ = gpu_run(w, inp, logits_override=[lg])
    r = oracle.route(lg.astype(np.float64), w.k)
    for k in ("topk_idx", "counts", "offsets", "row_of_slot", "src_of_row"):
        assert np.array_equal(gres[0][k], r[k]), k
    assert_close("topk_w", gres[0]["topk_w"], r["topk_w"], TOL_ROUTING)


def test_microbatch_accumulation_small():
    w = small_workload(513, 128, 16, 4, 128, BF16, "zipf", seed=34, n_empty=2, micro_T=(300, 77, 0, 513))
    inp = make_inputs(w)
    gres, gacc = gpu_run(w, inp)
    ores, oacc = oracle_run(w, inp)
    compare(w, gres, gacc, ores, oacc)
    assert gres[2]["dw_unchanged"]


def test_router_bf16_full():
    """bf16, T=4096 d=1024 E=8 top-2 F=2816, one expert emptied by the router bias."""
    w = WORKLOADS["router_bf16"]
    inp = make_inputs(w)
    gres, gacc = gpu_run(w, inp)
    ores, oacc = oracle_run(w, inp)
    errs = compare(w, gres, gacc, ores, oacc)
    assert 0 in gres[0]["counts"].tolist()
    print("router_bf16 errors:", {k: f"{v:.2e}" for k, v in errs.items()})


def test_sentinels_every_row_written():
    w = small_workload(421, 128, 8, 2, 192, BF16, "zipf", seed=35, n_empty=1)
    inp = make_inputs(w)
    gres, _ = gpu_run(w, inp, sentinel=True)
    g = gres[0]
    for k in ("x_perm", "h", "a", "y", "out", "dy", "dx_perm", "dx", "topk_w", "dtopk_w", "dlogits"):
        assert np.all(np.isfinite(g[k])), f"{k} has unwritten entries"
    assert np.all(g["topk_idx"] >= 0) and np.all(g["src_of_row"] >= 0)


def test_determinism_bitwise():
    w = small_workload(1500, 256, 16, 4, 128, BF16, "zipf", seed=36, n_empty=2)
    inp = make_inputs(w)
    a, aa = gpu_run(w, inp)
    b, bb = gpu_run(w, inp)
    for k in a[0]:
        assert np.array_equal(a[0][k], b[0][k], equal_nan=True), k
    for k in aa:
        assert np.array_equal(aa[k], bb[k]), k


def test_empty_microbatch_no_launch_no_write():
    import torch
    m, MoeLayer = _moe()
    layer = MoeLayer(16, 64, 4, 2, 64, m.MOE_DTYPE_BF16)
    for name in ("x_perm", "h", "y", "out", "dx"):
        getattr(layer, name).fill_(3.0)
    layer.counts.fill_(-5)
    s = layer.shape(0)
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    # every entry point accepts NULLs and writes nothing for T = 0
    m.moe_route(s, None, None, None, None, None, None, None, None, None, None, None, 0)
    m.moe_permute(s, None, None, None)
    m.moe_grouped_gemm_fwd(s, None, None, None, None, None, None, None, None, 0)
    m.moe_unpermute_combine(s, None, None, None, None)
    m.moe_unpermute_combine_bwd(s, None, None, None, None, None, None)
    m.moe_route_bwd(s, None, None, None, None, None, None, None, None, None, None, 0)
    m.moe_grouped_gemm_bwd(s, None, None, None, None, None, None, None, None, None, None, None, 0)
    m.moe_permute_bwd(s, None, None, None, None)
    layer.forward(0, x, x, x, logits=torch.empty(0, 4, device="cuda"))
    torch.cuda.synchronize()
    for name in ("x_perm", "h", "y", "out", "dx"):
        assert torch.all(getattr(layer, name).float() == 3.0), name
    assert torch.all(layer.counts == -5)


def test_workspace_reuse_across_sizes():
    """One workspace sized for the largest microbatch serves smaller ones."""
    w = small_workload(900, 128, 8, 2, 128, BF16, "zipf", seed=37, n_empty=1, micro_T=(900, 5, 450, 1))
    inp = make_inputs(w)
    gres, gacc = gpu_run(w, inp)
    ores, oacc = oracle_run(w, inp)
    compare(w, gres, gacc, ores, oacc)


# --- activation recompute (MOE_FLAG_RECOMPUTE) and no-grad forward ---------

RECOMPUTE_CASES = [c for c in SMALL_CASES if c[0] in (
    "tiny_f32_router", "bf16_ragged_tiles_zipf", "bf16_renorm_k8", "f32_zipf", "bf16_E256_k16", "bf16_single_expert")]
# and the first wide random shapes (both dtypes, renorm, E up to 255, d up to 1024)
RECOMPUTE_CASES += RANDOM_WIDE_CASES[:8]


def _assert_bitwise(a_res, a_acc, b_res, b_acc):
    for i, (ra, rb) in enumerate(zip(a_res, b_res)):
        for k in ra:
            if ra[k] is None or rb[k] is None:
                continue
            assert np.array_equal(ra[k], rb[k], equal_nan=True), f"mb{i} {k} differs from the saved-activation run"
    for k in a_acc:
        assert np.array_equal(a_acc[k], b_acc[k]), f"{k} differs from the saved-activation run"


@pytest.mark.parametrize("name,w,renorm", RECOMPUTE_CASES, ids=[c[0] for c in RECOMPUTE_CASES])
def test_recompute_small(name, w, renorm):
    """The recomputing backward matches the oracle to the bar and the
    saved-activation path bit for bit (same kernels, same order)."""
    print(f"[recompute] {name} T={w.T} d={w.d} E={w.E} k={w.k} F={w.F} {w.dtype}", flush=True)
    inp = make_inputs(w)
    gres, gacc = gpu_run(w, inp, renorm, recompute=True)
    ores, oacc = oracle_run(w, inp, renorm)
    compare(w, gres, gacc, ores, oacc, renorm)
    sres, sacc = gpu_run(w, inp, renorm)
    _assert_bitwise(gres, gacc, sres, sacc)


def test_recompute_microbatch_accumulation():
    """Microbatches T = 300, 77, 0, 513 on one recomputing layer: dW
    accumulate, the empty microbatch leaves them bit-identical."""
    w = small_workload(513, 128, 16, 4, 128, BF16, "zipf", seed=34, n_empty=2, micro_T=(300, 77, 0, 513))
    inp = make_inputs(w)
    gres, gacc = gpu_run(w, inp, recompute=True)
    ores, oacc = oracle_run(w, inp)
    compare(w, gres, gacc, ores, oacc)
    assert gres[2]["dw_unchanged"]
    sres, sacc = gpu_run(w, inp)
    _assert_bitwise(gres, gacc, sres, sacc)


def test_nograd_forward():
    """Forward alone (no backward) under recompute, twice in a row on a
    smaller then larger microbatch: out matches the oracle and the
    saved-activation forward bit for bit; the layer owns no h or a."""
    import torch
    m, MoeLayer = _moe()
    w = small_workload(700, 256, 8, 2, 192, BF16, "zipf", seed=38, n_empty=1, micro_T=(300, 700))
    inp = make_inputs(w)
    W = inp["weights"]
    wgu, wdn = to_device(W["w_gu"], BF16), to_device(W["w_down"], BF16)
    lay_rc = MoeLayer(700, w.d, w.E, w.k, w.F, m.MOE_DTYPE_BF16, recompute=True)
    lay_sv = MoeLayer(700, w.d, w.E, w.k, w.F, m.MOE_DTYPE_BF16)
    assert lay_rc.h is None and lay_rc.a is None
    for mb in inp["micro"]:
        T = mb["x"].shape[0]
        x, lg = to_device(mb["x"], BF16), to_device(mb["logits"], F32)
        o_rc = lay_rc.forward(T, x, wgu, wdn, logits=lg).out.clone()
        o_sv = lay_sv.forward(T, x, wgu, wdn, logits=lg).out.clone()
        torch.cuda.synchronize()
        assert torch.equal(o_rc, o_sv)
        assert torch.equal(lay_rc.fwd_a_view(T), lay_sv.a[:T * w.k])
        out, _ = oracle.layer_fwd(to_f64(mb["x"], BF16), to_f64(W["w_gu"], BF16), to_f64(W["w_down"], BF16), w.k,
                                  logits=mb["logits"].astype(np.float64))
        assert_close("out (no-grad)", to_host64(o_rc), out, TOL[BF16])
