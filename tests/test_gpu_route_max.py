"""Routing at the largest token count the library accepts.

T = 2^24 - 1 tokens (the per-launch thread bound: T * 256 < 2^32) over
E = 8 experts, top-2: 33.5 M slots, 262,144 top-k workgroups, a per-expert
scan over as many workgroup histograms, and row indices up to 2^25. The
whole tables (topk_idx, counts, offsets, row_of_slot, src_of_row) are
compared bit for bit with the fp64 oracle's selection and stable counting
sort (top-k by logit, ties to the lower id, rows of one expert in source
order; Support combined expert and data parallelism in TrainerRank, Desired
behavior), the weights within 1e-4, and the routing backward's dlogits
within 1e-4 on every row. The logits are seeded draws made on the device
with torch's generator, rounded to multiples of 1/8 so that ties occur.
"""
import numpy as np
import pytest

import oracle
from tests.parity_util import TOL_ROUTING, assert_close

pytestmark = pytest.mark.gpu

T, E, K = (1 << 24) - 1, 8, 2


def test_route_largest_token_count():
    import torch
    import token_dispatch_grouped_amd as m
    print(f"[route-max] T={T} E={E} k={K}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(2024)
    lg = (torch.randn(T, E, generator=g, device="cuda", dtype=torch.float32) * 8).round() / 8
    # a bf16 layer (the routing itself runs on fp32 logits either way); an fp32 layer of
    # this size is refused, its grouped GEMM grid would pass 2^32 threads
    s = m.make_shape(T, 64, E, K, 64, m.MOE_DTYPE_BF16, 0)
    rws, _, _ = m.moe_workspace_size(s)
    ws = torch.empty(rws, dtype=torch.uint8, device="cuda")
    i32 = torch.int32
    idx = torch.full((T, K), -7, dtype=i32, device="cuda")
    tw = torch.full((T, K), float("nan"), dtype=torch.float32, device="cuda")
    counts = torch.full((E,), -7, dtype=i32, device="cuda")
    offs = torch.full((E + 1,), -7, dtype=i32, device="cuda")
    ros = torch.full((T, K), -7, dtype=i32, device="cuda")
    sor = torch.full((T * K,), -7, dtype=i32, device="cuda")
    m.moe_route(s, None, None, None, lg, idx, tw, counts, offs, ros, sor, ws, ws.numel())
    dtw = torch.randn(T, K, generator=g, device="cuda", dtype=torch.float32)
    dl = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda")
    m.moe_route_bwd(s, dtw, lg, idx, tw, None, None, dl, None, None, ws, ws.numel())
    torch.cuda.synchronize()

    lg64 = lg.cpu().numpy().astype(np.float64)
    ref = oracle.route(lg64, K)
    for name, got in (("topk_idx", idx), ("counts", counts), ("offsets", offs), ("row_of_slot", ros),
                      ("src_of_row", sor)):
        assert np.array_equal(got.cpu().numpy(), ref[name].reshape(tuple(got.shape))), name
    assert_close("topk_w", tw.cpu().numpy(), ref["topk_w"], TOL_ROUTING)
    del idx, ros, sor
    want = oracle.route_bwd(dtw.cpu().numpy().astype(np.float64), lg64, ref["topk_idx"], ref["topk_w"])
    assert_close("dlogits", dl.cpu().numpy(), want, TOL_ROUTING)
