"""moe_route_noalloc (routing with the library's static per-GPU scratch, no
workspace) gives bit for bit what moe_route gives with a workspace, on two
calls in a row on one GPU, the second with fewer tokens (the scratch keeps
the first call's histograms, which the second must not use), and in router
mode. Run after the other GPU tests and alone in a fresh process alike."""
import numpy as np
import pytest

from tests.parity_util import to_device
from workloads import BF16, F32, make_inputs, small_workload

pytestmark = pytest.mark.gpu

KEYS = ("logits", "topk_idx", "topk_w", "counts", "offsets", "row_of_slot", "src_of_row")


def _buffers(T, E, k):
    import torch
    f32, i32 = torch.float32, torch.int32
    return dict(logits=torch.full((T, E), float("nan"), dtype=f32, device="cuda"),
                topk_idx=torch.full((T, k), -7, dtype=i32, device="cuda"),
                topk_w=torch.full((T, k), float("nan"), dtype=f32, device="cuda"),
                counts=torch.full((E,), -7, dtype=i32, device="cuda"),
                offsets=torch.full((E + 1,), -7, dtype=i32, device="cuda"),
                row_of_slot=torch.full((T, k), -7, dtype=i32, device="cuda"),
                src_of_row=torch.full((T * k,), -7, dtype=i32, device="cuda"))


def _route_both(w, T, logits=None, x=None, wr=None, bias=None):
    """The same routing through moe_route (workspace) and moe_route_noalloc."""
    import torch
    import token_dispatch_grouped_amd as m
    dt = m.MOE_DTYPE_BF16 if w.dtype == BF16 else m.MOE_DTYPE_F32
    s = m.make_shape(T, w.d, w.E, w.k, w.F, dt, 0)
    rws, _, _ = m.moe_workspace_size(s)
    ws = torch.empty(max(rws, 256), dtype=torch.uint8, device="cuda")
    a, b = _buffers(T, w.E, w.k), _buffers(T, w.E, w.k)
    if logits is not None:
        a["logits"].copy_(logits)
        b["logits"].copy_(logits)
    m.moe_route(s, x, wr, bias, a["logits"], a["topk_idx"], a["topk_w"], a["counts"], a["offsets"],
                a["row_of_slot"], a["src_of_row"], ws, ws.numel())
    m.moe_route_noalloc(s, x, wr, bias, b["logits"], b["topk_idx"], b["topk_w"], b["counts"], b["offsets"],
                        b["row_of_slot"], b["src_of_row"])
    torch.cuda.synchronize()
    return a, b


def _assert_same(a, b, what):
    import torch
    for k in KEYS:
        assert torch.equal(a[k], b[k]), f"{what}: {k} differs between moe_route and moe_route_noalloc"
    assert int(a["counts"].sum()) == a["src_of_row"].numel()


def test_route_noalloc_matches_route_two_calls():
    import torch
    # first call: 9000 tokens over 64 experts (36 workgroups of histograms),
    # second: 700 tokens over the same experts, then a 1-token call
    w = small_workload(9000, 64, 64, 8, 64, BF16, "zipf", seed=71, n_empty=5)
    lg = to_device(np.ascontiguousarray(make_inputs(w)["micro"][0]["logits"]), F32)
    print("[no-alloc] T=9000 E=64 k=8 then T=700 then T=1", flush=True)
    for T in (9000, 700, 1):
        a, b = _route_both(w, T, logits=lg[:T])
        _assert_same(a, b, f"T={T}")
    # router mode on a second shape (E = 8, top-2), larger then smaller
    w2 = small_workload(3000, 256, 8, 2, 64, BF16, "router", seed=72, n_empty=1)
    inp = make_inputs(w2)
    x = to_device(inp["micro"][0]["x"], BF16)
    wr = to_device(inp["weights"]["w_router"], BF16)
    bias = to_device(inp["weights"]["bias"], F32)
    for T in (3000, 257):
        a, b = _route_both(w2, T, x=x[:T].contiguous(), wr=wr, bias=bias)
        _assert_same(a, b, f"router T={T}")
