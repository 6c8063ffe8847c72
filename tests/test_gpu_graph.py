"""A layer step captured in a HIP graph replays bit for bit.

Every entry point is stream-ordered work only: no allocation, no host
synchronisation, no device-to-host read, and no memset node (the kernels
write every byte they own). So one forward + backward of the layer (routing
on given logits, permute, grouped GEMMs, combine and their backward) can be
captured once with torch.cuda.graph and replayed. Each replay must give
exactly what the eager step gave. Between replays the program does eager
work of its own: it zeroes the weight gradients (which accumulate), fills
every output with NaN, runs a differently shaped layer step, and
synchronises. Three replays are checked.
"""
import numpy as np
import pytest

from tests.parity_util import to_device
from workloads import BF16, make_inputs, small_workload

pytestmark = pytest.mark.gpu

OUTS = ("out", "dx", "dlogits", "dy", "dx_perm", "topk_idx", "topk_w", "counts", "offsets", "row_of_slot",
        "src_of_row", "x_perm", "y")


def _setup(w, inp):
    import torch
    import token_dispatch_grouped_amd as m
    from token_dispatch_grouped_amd.layer import MoeLayer
    layer = MoeLayer(w.T, w.d, w.E, w.k, w.F, m.MOE_DTYPE_BF16)
    W = inp["weights"]
    mb = inp["micro"][0]
    t = dict(wgu=to_device(W["w_gu"], BF16), wdn=to_device(W["w_down"], BF16), x=to_device(mb["x"], BF16),
             dout=to_device(mb["dout"], BF16),
             dw_gu=torch.zeros(w.E, 2 * w.F, w.d, dtype=torch.float32, device="cuda"),
             dw_down=torch.zeros(w.E, w.d, w.F, dtype=torch.float32, device="cuda"))
    # the logits live in the layer's own buffer, so the step itself copies nothing
    layer.logits[:w.T].copy_(to_device(np.ascontiguousarray(mb["logits"], dtype=np.float32), "f32"))
    return layer, t


def _step(w, layer, t):
    layer.forward(w.T, t["x"], t["wgu"], t["wdn"])
    layer.backward(w.T, t["dout"], t["wgu"], t["wdn"], t["dw_gu"], t["dw_down"])


def _snapshot(layer, t):
    import torch
    torch.cuda.synchronize()
    snap = {n: getattr(layer, n).clone().cpu() for n in OUTS}
    snap["dw_gu"] = t["dw_gu"].clone().cpu()
    snap["dw_down"] = t["dw_down"].clone().cpu()
    return snap


def _poison(layer, t):
    import torch
    for n in OUTS:
        buf = getattr(layer, n)
        if buf.is_floating_point():
            buf.fill_(float("nan"))
        else:
            buf.fill_(-7)
    t["dw_gu"].zero_()
    t["dw_down"].zero_()
    torch.cuda.synchronize()


def test_layer_step_graph_replays_bitwise():
    import torch
    w = small_workload(1500, 256, 16, 4, 192, BF16, "zipf", seed=81, n_empty=3)
    wo = small_workload(700, 384, 8, 2, 256, BF16, "normal", seed=82)
    print(f"[graph] T={w.T} d={w.d} E={w.E} k={w.k} F={w.F}; other step T={wo.T} d={wo.d}", flush=True)
    inp, inpo = make_inputs(w), make_inputs(wo)
    layer, t = _setup(w, inp)
    other, to = _setup(wo, inpo)

    _step(w, layer, t)
    ref = _snapshot(layer, t)
    assert torch.isfinite(ref["out"].float()).all() and int(ref["counts"].sum()) == w.T * w.k

    # capture on a side stream (torch.cuda.graph makes it current), after a warm-up step there
    _poison(layer, t)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(w, layer, t)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(w, layer, t)
    torch.cuda.synchronize()

    for rep in range(3):
        _poison(layer, t)
        _step(wo, other, to)  # the program's own eager work between replays
        torch.cuda.synchronize()
        g.replay()
        got = _snapshot(layer, t)
        for name, want in ref.items():
            assert torch.equal(got[name].view(torch.uint8) if got[name].is_floating_point() else got[name],
                               want.view(torch.uint8) if want.is_floating_point() else want), \
                f"replay {rep}: {name} differs from the eager step"
