"""Float64 CPU oracle of expert-parallel token exchange around the MoE layer:
the send plan of each source rank, the exchange of counts and rows between
ranks, the regrouping of received rows into local-expert-contiguous order,
and the way back.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests, the smoke
check and the bench's CPU-baseline leg may use it.

What the pages fix and what is read into them
---------------------------------------------
"Support combined expert and data parallelism in TrainerRank" asks for
expert parallelism (EP > 1) combined with data parallelism, where ranks hold
different token counts, uneven work or none at all (Desired behavior), with
expert communication, collective ordering and buffer capacity coordinated
inside the runtime, callers never padding, and outputs back in full source
order (same section); its Acceptance section asks for an EP=2 canary on
unequal batches including an empty-work case. The pages give no algorithm
for the exchange. The readings taken here are the plainest ones:

* the global experts are split into EP contiguous blocks of E_local: global
  expert g = r * E_local + e is local expert e of rank r;
* every source rank routes its own tokens over all EP * E_local experts with
  the single-rank routing rule (oracle.moe.route), so its dispatched rows
  x_perm are already grouped by destination rank: the segment for rank r is
  rows [offsets[r E_local], offsets[(r+1) E_local]), ordered by local expert,
  then by source token;
* send plan: send_counts[r, e] = counts[r E_local + e] and
  send_offsets[r] = offsets[r E_local], send_offsets[EP] = T k; a rank with
  T = 0 still has its (all-zero) table, since every rank enters the counts
  exchange whatever its work;
* counts exchange: rank r receives recv_counts[s, e] = send_counts_s[r, e]
  from every source s;
* rows exchange: rank r's receive buffer holds the segments of sources
  0, 1, ..., EP-1 one after the other (recv_offsets[s] = rows of the
  sources before s), each in its own order;
* regroup: the grouped FFN needs local-expert-contiguous rows, so rank r
  orders its rows by local expert, then by source rank, then by their order
  in the source's segment; regroup_row[i] is the grouped row of received
  row i; local_counts[e] = sum over s of recv_counts[s, e];
* the expert FFN runs on the grouped rows (oracle.moe.expert_ffn_fwd/_bwd),
  rows return by the inverse regroup and the reverse exchange, and every
  source combines its own tokens (oracle.moe.unpermute_combine) in full
  source order. The backward takes the same path with dY out and dX_perm
  back; the weight gradient of an expert sums the rows of every source.

With these readings the whole exchange is a permutation of rows, so every
source's outputs and gradients equal those of the single-rank layer over
all EP * E_local experts, which is what the tests pin it to.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np

from . import moe as _moe

__all__ = ["ep_send_plan", "ep_send_plan_empty", "ep_recv_plan", "ep_exchange", "ep_return", "ep_regroup", "ep_ungroup",
           "ep_layer_fwd", "ep_layer_bwd"]


def ep_send_plan(counts: np.ndarray, offsets: np.ndarray, ep: int, T: int):
    """(send_counts [ep, E_local] int32, send_offsets [ep+1] int32) of one
    source rank from its global-expert counts and offsets; all zeros when
    T = 0 (counts and offsets are then not read)."""
    E = len(counts)
    assert E % ep == 0
    e_local = E // ep
    if T == 0:
        return ep_send_plan_empty(ep, e_local)
    send_counts = np.asarray(counts, dtype=np.int32).reshape(ep, e_local).copy()
    send_offsets = np.array([offsets[r * e_local] for r in range(ep)] + [offsets[E]], dtype=np.int32)
    return send_counts, send_offsets


def ep_send_plan_empty(ep: int, e_local: int):
    """The plan of a rank with no tokens: all-zero counts and offsets."""
    return np.zeros((ep, e_local), dtype=np.int32), np.zeros(ep + 1, dtype=np.int32)


def ep_recv_plan(recv_counts: np.ndarray) -> Dict[str, np.ndarray]:
    """Receive plan of one destination rank from recv_counts [EP, E_local]
    (row s: what source s sends it).

    Received rows are numbered source-major (source s's segment in its own
    order: local expert, then source token); the grouped order is local
    expert, then source, then that order. Returns local_counts [E_local],
    local_offsets [E_local+1], recv_offsets [EP+1] and regroup_row [R_recv]
    (the grouped row of each received row)."""
    rc = np.asarray(recv_counts, dtype=np.int64)
    ep, e_local = rc.shape
    local_counts = rc.sum(axis=0)
    local_offsets = np.concatenate([[0], np.cumsum(local_counts)])
    recv_offsets = np.concatenate([[0], np.cumsum(rc.sum(axis=1))])
    R = int(recv_offsets[-1])
    regroup_row = np.empty(R, dtype=np.int64)
    i = 0  # received row, walking source-major
    for s in range(ep):
        for e in range(e_local):
            n = int(rc[s, e])
            # grouped rows of expert e: sources before s come first
            start = int(local_offsets[e] + rc[:s, e].sum())
            regroup_row[i:i + n] = np.arange(start, start + n)
            i += n
    assert i == R
    return {"local_counts": local_counts.astype(np.int32), "local_offsets": local_offsets.astype(np.int32),
            "recv_offsets": recv_offsets.astype(np.int32), "regroup_row": regroup_row.astype(np.int32)}


def ep_exchange(send_bufs: List[np.ndarray], send_offsets: List[np.ndarray],
                recv_offsets: List[np.ndarray]) -> List[np.ndarray]:
    """Rows from every source to every destination: destination r's buffer
    holds, at rows recv_offsets[r][s] on, rows send_offsets[s][r] ..
    send_offsets[s][r+1] of source s's buffer."""
    ep = len(send_bufs)
    tail = send_bufs[0].shape[1:]
    out = []
    for r in range(ep):
        buf = np.zeros((int(recv_offsets[r][-1]),) + tail)
        for s in range(ep):
            a, b = int(send_offsets[s][r]), int(send_offsets[s][r + 1])
            buf[recv_offsets[r][s]:recv_offsets[r][s] + (b - a)] = send_bufs[s][a:b]
        out.append(buf)
    return out


def ep_return(recv_bufs: List[np.ndarray], send_offsets: List[np.ndarray], recv_offsets: List[np.ndarray],
              rows_per_source: List[int]) -> List[np.ndarray]:
    """The reverse exchange: source s gets back, at its rows
    send_offsets[s][r] .., what destination r holds at recv_offsets[r][s] .."""
    ep = len(recv_bufs)
    tail = recv_bufs[0].shape[1:]
    out = []
    for s in range(ep):
        buf = np.zeros((rows_per_source[s],) + tail)
        for r in range(ep):
            a, b = int(send_offsets[s][r]), int(send_offsets[s][r + 1])
            buf[a:b] = recv_bufs[r][recv_offsets[r][s]:recv_offsets[r][s] + (b - a)]
        out.append(buf)
    return out


def ep_regroup(recv: np.ndarray, regroup_row: np.ndarray) -> np.ndarray:
    """grouped[regroup_row[i]] = recv[i]."""
    out = np.zeros_like(recv)
    out[regroup_row] = recv
    return out


def ep_ungroup(grouped: np.ndarray, regroup_row: np.ndarray) -> np.ndarray:
    """recv[i] = grouped[regroup_row[i]]."""
    return grouped[regroup_row]


def ep_layer_fwd(xs, logits, w_gu, w_down, k, ep, renorm=False):
    """Forward of EP ranks exchanging tokens: xs[s] [T_s, d] and logits[s]
    [T_s, E] of every source rank (T_s may be 0); w_gu / w_down hold all
    E = ep * E_local experts (rank r owns [r E_local, (r+1) E_local)).
    Returns (outs per source, saved) where saved keeps every step's tables and
    buffers."""
    E = w_gu.shape[0]
    e_local = E // ep
    d = w_gu.shape[2]
    routes, send_counts, send_offsets, x_perms, Ts = [], [], [], [], []
    for s in range(ep):
        T = xs[s].shape[0]
        Ts.append(T)
        if T:
            r = _moe.route(logits[s], k, renorm)
            sc, so = ep_send_plan(r["counts"], r["offsets"], ep, T)
            xp = _moe.permute(xs[s], r["row_of_slot"])
        else:
            r = None
            sc, so = ep_send_plan(np.zeros(E, dtype=np.int32), None, ep, 0)
            xp = np.zeros((0, d))
        routes.append(r)
        send_counts.append(sc)
        send_offsets.append(so)
        x_perms.append(xp)
    # counts exchange, then every destination's receive plan
    recv_counts = [np.stack([send_counts[s][r] for s in range(ep)]) for r in range(ep)]
    plans = [ep_recv_plan(rc) for rc in recv_counts]
    recv_offsets = [p["recv_offsets"] for p in plans]
    recv_x = ep_exchange(x_perms, send_offsets, recv_offsets)
    grouped_x, hs, as_, ys_grouped, recv_y = [], [], [], [], []
    for r in range(ep):
        gx = ep_regroup(recv_x[r], plans[r]["regroup_row"])
        h, a, y = _moe.expert_ffn_fwd(gx, w_gu[r * e_local:(r + 1) * e_local],
                                      w_down[r * e_local:(r + 1) * e_local], plans[r]["local_offsets"])
        grouped_x.append(gx)
        hs.append(h)
        as_.append(a)
        ys_grouped.append(y)
        recv_y.append(ep_ungroup(y, plans[r]["regroup_row"]))
    y_perms = ep_return(recv_y, send_offsets, recv_offsets, [T * k for T in Ts])
    outs = []
    for s in range(ep):
        if Ts[s]:
            outs.append(_moe.unpermute_combine(y_perms[s], routes[s]["topk_w"], routes[s]["row_of_slot"]))
        else:
            outs.append(np.zeros((0, d)))
    saved = dict(routes=routes, send_counts=send_counts, send_offsets=send_offsets, recv_counts=recv_counts,
                 plans=plans, x_perms=x_perms, recv_x=recv_x, grouped_x=grouped_x, h=hs, a=as_, y_grouped=ys_grouped,
                 y_perms=y_perms, logits=logits, Ts=Ts, ep=ep, e_local=e_local, k=k, renorm=renorm)
    return outs, saved


def ep_layer_bwd(douts, saved, w_gu, w_down):
    """Backward of ep_layer_fwd: per source dy (in its x_perm layout), dtopk_w,
    dlogits and dx; per destination the grouped dh and dx rows; the weight
    gradients of all E experts (each summing the rows of every source)."""
    ep, e_local, k = saved["ep"], saved["e_local"], saved["k"]
    d = w_gu.shape[2]
    dys, dtws, dlogits = [], [], []
    for s in range(ep):
        r = saved["routes"][s]
        if saved["Ts"][s]:
            dy, dtw = _moe.unpermute_combine_bwd(douts[s], saved["y_perms"][s], r["topk_w"], r["row_of_slot"])
            dl = _moe.route_bwd(dtw, saved["logits"][s], r["topk_idx"], r["topk_w"], saved["renorm"])
        else:
            dy, dtw, dl = np.zeros((0, d)), np.zeros((0, k)), np.zeros((0, w_gu.shape[0]))
        dys.append(dy)
        dtws.append(dtw)
        dlogits.append(dl)
    recv_offsets = [p["recv_offsets"] for p in saved["plans"]]
    recv_dy = ep_exchange(dys, saved["send_offsets"], recv_offsets)
    dw_gu = np.zeros_like(w_gu, dtype=np.float64)
    dw_down = np.zeros_like(w_down, dtype=np.float64)
    recv_dx, grouped_dh = [], []
    for r in range(ep):
        plan = saved["plans"][r]
        gdy = ep_regroup(recv_dy[r], plan["regroup_row"])
        sl = slice(r * e_local, (r + 1) * e_local)
        gdx, dwg, dwd, dh = _moe.expert_ffn_bwd(gdy, saved["grouped_x"][r], saved["h"][r], saved["a"][r],
                                                w_gu[sl], w_down[sl], plan["local_offsets"])
        dw_gu[sl] = dwg
        dw_down[sl] = dwd
        grouped_dh.append(dh)
        recv_dx.append(ep_ungroup(gdx, plan["regroup_row"]))
    dx_perms = ep_return(recv_dx, saved["send_offsets"], recv_offsets, [T * k for T in saved["Ts"]])
    dxs = []
    for s in range(ep):
        if saved["Ts"][s]:
            dxs.append(_moe.permute_bwd(dx_perms[s], saved["routes"][s]["row_of_slot"]))
        else:
            dxs.append(np.zeros((0, d)))
    return dict(dy=dys, dtopk_w=dtws, dlogits=dlogits, dx_perm=dx_perms, dx=dxs, dw_gu=dw_gu, dw_down=dw_down,
                grouped_dh=grouped_dh)
