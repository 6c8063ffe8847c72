"""Routing over every split of a logit row across lanes.

The top-k and the routing backward give each token's row to 1, 2, 4 or 8
lanes, which hold at most 8, 16 or 32 logits each: 16-byte chunks when E is a
multiple of 4, single values otherwise. Each E below sits on one side of a
boundary of that split. Per E, a few k over T = 333 tokens (five full
64-token workgroups and a ragged sixth) are compared with the fp64 oracle
(top-k by logit, ties to the lower expert id, softmax weights, stable rows;
Support combined expert and data parallelism in TrainerRank, Desired
behavior):
  * the tables (topk_idx, counts, offsets, row_of_slot, src_of_row) bit for
    bit, and topk_w within 1e-4 (fp32 arithmetic on fp32 logits);
  * dlogits of the routing backward within 1e-4, with and without
    renormalisation, overwritten and accumulated onto a seeded array.
Half the rows hold logits from two integer levels, so most tokens carry ties.
A further pass per k puts -inf, NaN, -0.0 and +inf into four rows of the last
workgroup (tables bit for bit; weights except on the row whose maximum is
infinite, where both sides give exp(inf - inf)).
"""
import numpy as np
import pytest

import oracle
from tests.parity_util import TOL_ROUTING, assert_close
from workloads import tie_logits

pytestmark = pytest.mark.gpu

T = 333
E_VALUES = [1, 3, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200, 255, 256]


def _k_values(E):
    return sorted({1, min(E, 3), min(E, 8), min(E, 16)})


def _logits(E, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ties = tie_logits(T, E, seed + 1, levels=2)
    lg[::2] = ties[::2]
    return lg


def _route(E, k, lg, renorm):
    import torch
    import token_dispatch_grouped_amd as m
    flags = m.MOE_FLAG_RENORM if renorm else 0
    s = m.make_shape(T, 64, E, k, 64, m.MOE_DTYPE_F32, flags)
    rws, _, _ = m.moe_workspace_size(s)
    ws = torch.empty(max(rws, 256), dtype=torch.uint8, device="cuda")
    i32 = torch.int32
    out = dict(logits=torch.from_numpy(lg).cuda(),
               topk_idx=torch.full((T, k), -7, dtype=i32, device="cuda"),
               topk_w=torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda"),
               counts=torch.full((E,), -7, dtype=i32, device="cuda"),
               offsets=torch.full((E + 1,), -7, dtype=i32, device="cuda"),
               row_of_slot=torch.full((T, k), -7, dtype=i32, device="cuda"),
               src_of_row=torch.full((T * k,), -7, dtype=i32, device="cuda"))
    m.moe_route(s, None, None, None, out["logits"], out["topk_idx"], out["topk_w"], out["counts"],
                out["offsets"], out["row_of_slot"], out["src_of_row"], ws, ws.numel())
    torch.cuda.synchronize()
    return s, ws, out


def _route_bwd(s, ws, out, dtw, dlogits0, accumulate):
    import torch
    import token_dispatch_grouped_amd as m
    if accumulate:
        s = m.make_shape(s.T, s.d, s.E, s.k, s.F, s.dtype, s.flags | m.MOE_FLAG_ACCUMULATE_DLOGITS)
    dl = torch.from_numpy(dlogits0).cuda()
    m.moe_route_bwd(s, torch.from_numpy(dtw).cuda(), out["logits"], out["topk_idx"], out["topk_w"], None, None, dl,
                    None, None, ws, ws.numel())
    torch.cuda.synchronize()
    return dl.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("E", E_VALUES)
def test_route_tables_and_backward_every_lane_split(E):
    print(f"[route-lanes] E={E} k={_k_values(E)} T={T}", flush=True)
    for k in _k_values(E):
        for renorm in (False, True):
            lg = _logits(E, 1000 * E + 10 * k + renorm)
            s, ws, out = _route(E, k, lg, renorm)
            ref = oracle.route(lg.astype(np.float64), k, renorm=renorm)
            for key in ("topk_idx", "counts", "offsets", "row_of_slot", "src_of_row"):
                got = out[key].cpu().numpy()
                assert np.array_equal(got, ref[key].reshape(got.shape)), f"E={E} k={k} renorm={renorm}: {key}"
            assert_close(f"E={E} k={k} topk_w", out["topk_w"].cpu().numpy(), ref["topk_w"], TOL_ROUTING)

            rng = np.random.Generator(np.random.PCG64(E * 31 + k))
            dtw = rng.standard_normal((T, k)).astype(np.float32)
            d0 = rng.standard_normal((T, E)).astype(np.float32)
            want = oracle.route_bwd(dtw.astype(np.float64), lg.astype(np.float64), ref["topk_idx"], ref["topk_w"],
                                    renorm=renorm)
            got = _route_bwd(s, ws, out, dtw, np.full((T, E), np.nan, np.float32), accumulate=False)
            assert_close(f"E={E} k={k} renorm={renorm} dlogits", got, want, TOL_ROUTING)
            got = _route_bwd(s, ws, out, dtw, d0, accumulate=True)
            assert_close(f"E={E} k={k} renorm={renorm} dlogits accumulated", got, d0.astype(np.float64) + want,
                         TOL_ROUTING)

        if E >= 2:  # one non-finite value or signed zero per row, in the ragged last workgroup
            lg = _logits(E, 1000 * E + 10 * k + 7)
            lg[320, 0] = -np.inf
            lg[321, E - 1] = np.nan
            lg[322, E // 2] = -0.0
            lg[323, (E + 1) // 2 % E] = np.inf
            s, ws, out = _route(E, k, lg, False)
            ref = oracle.route(lg.astype(np.float64), k)
            for key in ("topk_idx", "counts", "offsets", "row_of_slot", "src_of_row"):
                got = out[key].cpu().numpy()
                assert np.array_equal(got, ref[key].reshape(got.shape)), f"E={E} k={k} non-finite: {key}"
            fin = np.ones(T, bool)
            fin[323] = False  # an infinite maximum: exp(inf - inf) on both sides
            assert_close(f"E={E} k={k} topk_w non-finite", out["topk_w"].cpu().numpy()[fin], ref["topk_w"][fin],
                         TOL_ROUTING)
