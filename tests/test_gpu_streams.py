"""Two layers on two streams at once give bit for bit what they give one
after the other.

The library keeps no state between calls beyond a device-properties cache,
and the persistent GEMM launches assume nothing about which workgroups share
the GPU with them; every reduction has a fixed order. So interleaving two
layers' calls on two streams, with no synchronisation between them, must not
change a single bit of either layer's outputs, gradients or routing tables.
"""
import numpy as np
import pytest

from tests.parity_util import to_device
from workloads import BF16, make_inputs, small_workload

pytestmark = pytest.mark.gpu

NAMES = ("out", "dx", "dlogits", "topk_idx", "row_of_slot", "offsets")


def _setup(w, inp):
    import torch
    import token_dispatch_grouped_amd as m
    from token_dispatch_grouped_amd.layer import MoeLayer
    layer = MoeLayer(w.T, w.d, w.E, w.k, w.F, m.MOE_DTYPE_BF16)
    W = inp["weights"]
    mb = inp["micro"][0]
    t = dict(wgu=to_device(W["w_gu"], BF16), wdn=to_device(W["w_down"], BF16), x=to_device(mb["x"], BF16),
             dout=to_device(mb["dout"], BF16),
             lg=to_device(np.ascontiguousarray(mb["logits"], dtype=np.float32), "f32"),
             dw_gu=torch.zeros(w.E, 2 * w.F, w.d, dtype=torch.float32, device="cuda"),
             dw_down=torch.zeros(w.E, w.d, w.F, dtype=torch.float32, device="cuda"))
    return layer, t


def _fwd(w, layer, t):
    layer.forward(w.T, t["x"], t["wgu"], t["wdn"], logits=t["lg"])


def _bwd(w, layer, t):
    layer.backward(w.T, t["dout"], t["wgu"], t["wdn"], t["dw_gu"], t["dw_down"])


def _snapshot(layer, t):
    import torch
    snap = {n: getattr(layer, n).clone() for n in NAMES}
    snap["dw_gu"] = t["dw_gu"].clone()
    snap["dw_down"] = t["dw_down"].clone()
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in snap.items()}


def test_two_layers_two_streams_bitwise():
    import torch
    # two different shapes, both with several persistent tiles per workgroup in some product
    wa = small_workload(3000, 512, 16, 4, 256, BF16, "zipf", seed=41, n_empty=2)
    wb = small_workload(2200, 768, 8, 2, 320, BF16, "normal", seed=42)
    print(f"[streams] A T={wa.T} d={wa.d} E={wa.E} k={wa.k} F={wa.F}; B T={wb.T} d={wb.d} E={wb.E} k={wb.k} "
          f"F={wb.F}", flush=True)
    ia, ib = make_inputs(wa), make_inputs(wb)

    # one after the other, on the current stream
    la, ta = _setup(wa, ia)
    lb, tb = _setup(wb, ib)
    _fwd(wa, la, ta)
    _bwd(wa, la, ta)
    _fwd(wb, lb, tb)
    _bwd(wb, lb, tb)
    ref_a, ref_b = _snapshot(la, ta), _snapshot(lb, tb)

    # interleaved on two default-priority streams, no synchronisation in between
    la2, ta2 = _setup(wa, ia)
    lb2, tb2 = _setup(wb, ib)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(sa):
        _fwd(wa, la2, ta2)
    with torch.cuda.stream(sb):
        _fwd(wb, lb2, tb2)
    with torch.cuda.stream(sa):
        _bwd(wa, la2, ta2)
    with torch.cuda.stream(sb):
        _bwd(wb, lb2, tb2)
    torch.cuda.synchronize()
    got_a, got_b = _snapshot(la2, ta2), _snapshot(lb2, tb2)

    for name, ref, got in (("A", ref_a, got_a), ("B", ref_b, got_b)):
        for k in ref:
            assert torch.equal(ref[k], got[k]), f"layer {name}: {k} differs when run beside another layer"
