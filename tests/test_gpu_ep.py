"""Expert-parallel ranks simulated on one GPU (token_dispatch_grouped_amd.ep,
through the C ABI) against the fp64 exchange oracle (oracle.ep), which is
itself pinned to the single-rank layer over all experts.

Bit-exact: every source's routing and send tables and dispatched rows, every
destination's received counts, receive plan, regroup map and grouped rows.
Within the bars (2e-2 bf16, 1e-4 fp32; routing weights 1e-4): every
destination's h, a and grouped y, every source's out, dx, dtopk_w and
dlogits, and every expert's weight gradients (an expert no source routes to
keeps exactly zero). Cases: uneven sources, an empty source, an empty local
expert, a destination that receives nothing, EP = 1..4, bf16 and fp32.
"""
import zlib

import numpy as np
import pytest

import oracle
from tests.parity_util import TOL, TOL_ROUTING, assert_close, to_device, to_host64
from workloads import BF16, F32, make_ep_inputs, to_f64

pytestmark = pytest.mark.gpu

CASES = [
    # name, ep, Ts, d, e_local, k, F, dtype, routing, n_empty
    ("ep2_uneven", 2, (300, 77), 256, 3, 2, 192, BF16, "normal", 0),
    ("ep2_empty_source", 2, (250, 0), 128, 4, 2, 128, BF16, "zipf", 1),
    ("ep3_empty_first_source_empty_expert", 3, (0, 120, 257), 128, 2, 3, 64, BF16, "zipf", 1),
    ("ep4_k4", 4, (64, 5, 190, 33), 192, 2, 4, 128, BF16, "normal", 0),
    ("ep2_f32", 2, (40, 91), 128, 3, 2, 64, F32, "normal", 0),
    ("ep1", 1, (333,), 128, 8, 2, 128, BF16, "zipf", 2),
    # one destination receives nothing: all of rank 1's experts are forced empty
    ("ep2_idle_destination", 2, (200, 150), 128, 2, 1, 64, BF16, "normal", 0),
    # a larger one: 16 global experts, several tiles per destination
    ("ep2_medium", 2, (2048, 1500), 1024, 8, 4, 512, BF16, "zipf", 2),
]


def _run(ep, Ts, d, e_local, k, F, dtype, inp, fused=True):
    import torch
    import token_dispatch_grouped_amd as m
    from token_dispatch_grouped_amd.ep import EpLoopback
    mdt = m.MOE_DTYPE_BF16 if dtype == BF16 else m.MOE_DTYPE_F32
    lay = EpLoopback(ep, max(max(Ts), 1), d, e_local, k, F, mdt, fused=fused)
    W = inp["weights"]
    wgu, wdn = to_device(W["w_gu"], dtype), to_device(W["w_down"], dtype)
    xs = [to_device(mb["x"], dtype) for mb in inp["micro"]]
    lgs = [to_device(np.ascontiguousarray(mb["logits"]), F32) for mb in inp["micro"]]
    douts = [to_device(mb["dout"], dtype) for mb in inp["micro"]]
    E = ep * e_local
    dw_gu = torch.zeros(E, 2 * F, d, dtype=torch.float32, device="cuda")
    dw_dn = torch.zeros(E, d, F, dtype=torch.float32, device="cuda")
    outs = lay.forward(Ts, xs, lgs, wgu, wdn)
    # grouped rows and FFN activations of the forward, before the backward reuses buffers
    fwd = [{key: to_host64(r[key]) for key in ("gx", "h", "a", "gy")} for r in lay.dst]
    torch.cuda.synchronize()
    outs = [to_host64(o) for o in outs]
    grads = lay.backward(douts, wgu, wdn, dw_gu, dw_dn)
    torch.cuda.synchronize()
    return lay, outs, fwd, [{k_: to_host64(v) for k_, v in g.items()} for g in grads], to_host64(dw_gu), to_host64(dw_dn)


# the unfused path (exchange in receive order, then moe_ep_regroup and back) on a few of the cases
UNFUSED = {"ep2_uneven", "ep3_empty_first_source_empty_expert", "ep2_f32"}
ALL = [c + (True,) for c in CASES] + [c + (False,) for c in CASES if c[0] in UNFUSED]


@pytest.mark.parametrize("name,ep,Ts,d,e_local,k,F,dtype,routing,n_empty,fused", ALL,
                         ids=[c[0] + ("" if c[-1] else "_unfused") for c in ALL])
def test_ep_loopback_matches_oracle(name, ep, Ts, d, e_local, k, F, dtype, routing, n_empty, fused):
    print(f"[ep] {name} fused={fused}: ep={ep} T={Ts} d={d} E_local={e_local} k={k} F={F} {dtype}", flush=True)
    E = ep * e_local
    inp = make_ep_inputs(ep, Ts, d, e_local, k, F, dtype, seed=zlib.crc32(name.encode()) % 10_000, routing=routing,
                         n_empty=n_empty)
    if name == "ep2_idle_destination":  # every token routes to rank 0's experts
        for mb in inp["micro"]:
            mb["logits"][:, e_local:] = np.float32(-1e4)
    lay, outs, fwd, grads, dw_gu, dw_dn = _run(ep, Ts, d, e_local, k, F, dtype, inp, fused)
    W = inp["weights"]
    wgu64, wdn64 = to_f64(W["w_gu"], dtype), to_f64(W["w_down"], dtype)
    xs = [to_f64(mb["x"], dtype) for mb in inp["micro"]]
    lgs = [mb["logits"].astype(np.float64) for mb in inp["micro"]]
    douts = [to_f64(mb["dout"], dtype) for mb in inp["micro"]]
    o_outs, sv = oracle.ep_layer_fwd(xs, lgs, wgu64, wdn64, k, ep)
    og = oracle.ep_layer_bwd(douts, sv, wgu64, wdn64)
    tol = TOL[dtype]
    for s, T in enumerate(Ts):
        b = lay.src[s]
        assert np.array_equal(b["send_counts"].cpu().numpy().reshape(ep, e_local), sv["send_counts"][s]), (s, "send_counts")
        assert np.array_equal(b["send_offsets"].cpu().numpy(), sv["send_offsets"][s]), (s, "send_offsets")
        if T == 0:
            continue
        r = sv["routes"][s]
        for key in ("topk_idx", "counts", "offsets", "row_of_slot", "src_of_row"):
            assert np.array_equal(b[key][:len(r[key])].cpu().numpy(), r[key]), (s, key)
        assert_close(f"src{s} topk_w", to_host64(b["topk_w"][:T]), r["topk_w"], TOL_ROUTING)
        assert np.array_equal(to_host64(b["x_perm"][:T * k]), sv["x_perms"][s]), (s, "x_perm")
        assert_close(f"src{s} out", outs[s], o_outs[s], tol)
        for key in ("dx", "dtopk_w", "dlogits"):
            assert_close(f"src{s} {key}", grads[s][key], og[key][s], tol)
    for rr in range(ep):
        d_ = lay.dst[rr]
        p = sv["plans"][rr]
        R = int(p["recv_offsets"][-1])
        assert np.array_equal(d_["recv_counts"].cpu().numpy().reshape(ep, e_local), sv["recv_counts"][rr])
        for key in ("local_counts", "local_offsets", "recv_offsets"):
            assert np.array_equal(d_[key].cpu().numpy(), p[key]), (rr, key)
        assert np.array_equal(d_["regroup_row"][:R].cpu().numpy(), p["regroup_row"]), (rr, "regroup_row")
        assert np.array_equal(fwd[rr]["gx"][:R], sv["grouped_x"][rr]), (rr, "grouped x")
        if R:
            assert_close(f"dst{rr} h", fwd[rr]["h"][:R], sv["h"][rr], tol)
            assert_close(f"dst{rr} a", fwd[rr]["a"][:R], sv["a"][rr], tol)
            assert_close(f"dst{rr} y", fwd[rr]["gy"][:R], sv["y_grouped"][rr], tol)
    for e in range(E):
        for key, got in (("dw_gu", dw_gu), ("dw_down", dw_dn)):
            ref = og[key][e]
            if np.max(np.abs(ref)) == 0.0:
                assert np.all(got[e] == 0.0), f"{key}[{e}] of an expert nobody routes to is not exactly zero"
            else:
                assert_close(f"{key}[{e}]", got[e], ref, tol)
    if name == "ep2_idle_destination":
        assert int(sv["plans"][1]["recv_offsets"][-1]) == 0
