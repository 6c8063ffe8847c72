"""Expert-parallel ranks simulated on one GPU: buffers and call sequence.

EP ranks each hold their own tokens (any count, zero included) and E_local of
the EP * E_local experts. PyTorch only allocates device memory and provides
the stream; every step runs in the library's HIP kernels, in this order:

  forward, per source rank s : moe_route (all experts) -> moe_permute -> moe_ep_send_plan
  counts exchange             : moe_ep_exchange_counts_loopback
  per destination rank r      : moe_ep_recv_plan
  rows exchange               : moe_ep_exchange_loopback (rows land at their grouped rows)
  per destination rank r      : moe_grouped_gemm_fwd
  rows back                   : moe_ep_exchange_loopback (reverse, from the grouped rows)
  per source rank s           : moe_unpermute_combine

  backward, per source s      : moe_unpermute_combine_bwd -> moe_route_bwd
  rows exchange (dY)          : moe_ep_exchange_loopback (to the grouped rows)
  per destination r           : moe_grouped_gemm_bwd
  rows back (dX_perm)         : moe_ep_exchange_loopback (reverse)
  per source s                : moe_permute_bwd

The two exchange calls are the one-GPU stand-ins for the all-to-all of the
counts tables and the all-to-allv of the rows between real ranks. With
fused=False the rows land in receive order and moe_ep_regroup moves them to
the grouped order and back in separate passes (the form for an exchange that
cannot scatter, e.g. a collective all-to-allv). Every rank
takes part in every step in the same order whatever its token count, so an
empty rank never changes the sequence. Buffers are sized once for T_max
tokens per source; a destination can receive up to EP * T_max * k rows.
"""
from __future__ import annotations

from typing import List, Optional

import torch

from . import _lib as L
from .layer import torch_dtype


class EpLoopback:
    def __init__(self, ep: int, T_max: int, d: int, e_local: int, k: int, F: int, dtype: int = L.MOE_DTYPE_BF16,
                 renorm: bool = False, fused: bool = True, device: str = "cuda"):
        self.ep, self.T_max, self.d, self.e_local, self.k, self.F = ep, T_max, d, e_local, k, F
        self.fused = fused
        self.E = ep * e_local
        self.dtype = dtype
        self.flags = L.MOE_FLAG_RENORM if renorm else 0
        dev = torch.device(device)
        td = torch_dtype(dtype)
        f32, i32, u8 = torch.float32, torch.int32, torch.uint8
        R = T_max * k
        self.rows_cap = ep * R
        rws, _, _ = L.moe_workspace_size(self.src_shape(T_max))
        _, fws, bws = L.moe_workspace_size(self.dst_shape())
        # per source rank: routing tables, dispatched rows, combine results
        self.src = []
        for _ in range(ep):
            self.src.append(dict(
                route_ws=torch.empty(max(rws, 256), dtype=u8, device=dev),
                logits=torch.empty(T_max, self.E, dtype=f32, device=dev),
                topk_idx=torch.empty(T_max, k, dtype=i32, device=dev),
                topk_w=torch.empty(T_max, k, dtype=f32, device=dev),
                counts=torch.zeros(self.E, dtype=i32, device=dev),
                offsets=torch.zeros(self.E + 1, dtype=i32, device=dev),
                row_of_slot=torch.empty(T_max, k, dtype=i32, device=dev),
                src_of_row=torch.empty(R, dtype=i32, device=dev),
                send_counts=torch.zeros(self.E, dtype=i32, device=dev),
                send_offsets=torch.zeros(ep + 1, dtype=i32, device=dev),
                x_perm=torch.empty(R, d, dtype=td, device=dev),
                y_perm=torch.empty(R, d, dtype=td, device=dev),
                out=torch.empty(T_max, d, dtype=td, device=dev),
                dy=torch.empty(R, d, dtype=td, device=dev),
                dtopk_w=torch.empty(T_max, k, dtype=f32, device=dev),
                dlogits=torch.empty(T_max, self.E, dtype=f32, device=dev),
                dx_perm=torch.empty(R, d, dtype=td, device=dev),
                dx=torch.empty(T_max, d, dtype=td, device=dev)))
        # per destination rank: receive plan, received and grouped rows, FFN buffers
        cap = self.rows_cap
        self.dst = []
        for _ in range(ep):
            self.dst.append(dict(
                recv_counts=torch.zeros(self.E, dtype=i32, device=dev),
                local_counts=torch.zeros(e_local, dtype=i32, device=dev),
                local_offsets=torch.zeros(e_local + 1, dtype=i32, device=dev),
                recv_offsets=torch.zeros(ep + 1, dtype=i32, device=dev),
                regroup_row=torch.empty(cap, dtype=i32, device=dev),
                # received rows in receive order (x, then y, dy, dx); only without fusion
                recv=None if fused else torch.empty(cap, d, dtype=td, device=dev),
                gx=torch.empty(cap, d, dtype=td, device=dev),        # grouped x_perm
                h=torch.empty(cap, 2 * F, dtype=td, device=dev),
                a=torch.empty(cap, F, dtype=td, device=dev),
                gy=torch.empty(cap, d, dtype=td, device=dev),        # grouped y, then grouped dy
                gdx=torch.empty(cap, d, dtype=td, device=dev),
                fwd_ws=torch.empty(max(fws, 256), dtype=u8, device=dev),
                bwd_ws=torch.empty(max(bws, 256), dtype=u8, device=dev)))
        self.T: List[int] = [0] * ep

    def src_shape(self, T: int) -> L.moe_shape:
        return L.make_shape(T, self.d, self.E, self.k, self.F, self.dtype, self.flags)

    def dst_shape(self) -> L.moe_shape:
        """Grouped FFN of one destination: up to rows_cap rows over its E_local experts."""
        return L.make_shape(self.rows_cap, self.d, self.e_local, 1, self.F, self.dtype, 0)

    def _exchange(self, send_key: str, grouped_key: str, reverse: bool, stream=None):
        """Rows between the sources' send_key buffers and the destinations'
        grouped_key buffers; without fusion through the receive buffers and
        moe_ep_regroup."""
        ep = self.ep
        srcs = [s[send_key] for s in self.src]
        caps = [t * self.k for t in self.T]
        soffs = [s["send_offsets"] for s in self.src]
        roffs = [r["recv_offsets"] for r in self.dst]
        if self.fused:
            L.moe_ep_exchange_loopback(ep, self.d, self.dtype, srcs, caps, soffs, [r[grouped_key] for r in self.dst],
                                       [self.rows_cap] * ep, roffs, regroup_rows=[r["regroup_row"] for r in self.dst],
                                       reverse=reverse, stream=stream)
            return
        if reverse:
            for r in self.dst:
                L.moe_ep_regroup(self.d, self.dtype, self.rows_cap, ep, r["recv_offsets"], r["regroup_row"],
                                 r[grouped_key], r["recv"], reverse=True, stream=stream)
        L.moe_ep_exchange_loopback(ep, self.d, self.dtype, srcs, caps, soffs, [r["recv"] for r in self.dst],
                                   [self.rows_cap] * ep, roffs, reverse=reverse, stream=stream)
        if not reverse:
            for r in self.dst:
                L.moe_ep_regroup(self.d, self.dtype, self.rows_cap, ep, r["recv_offsets"], r["regroup_row"], r["recv"],
                                 r[grouped_key], reverse=False, stream=stream)

    def forward(self, Ts, xs, logits, w_gu, w_down, stream=None):
        """xs[s] [T_s, d], logits[s] [T_s, E] fp32 of every source; w_gu / w_down
        hold all E experts (rank r owns [r E_local, (r+1) E_local)). Returns the
        per-source outputs [T_s, d]."""
        self.T = [int(t) for t in Ts]
        ep, el = self.ep, self.e_local
        for s, (T, x, lg) in enumerate(zip(self.T, xs, logits)):
            b = self.src[s]
            sh = self.src_shape(T)
            if T:
                b["logits"][:T].copy_(lg)
            L.moe_route(sh, None, None, None, b["logits"], b["topk_idx"], b["topk_w"], b["counts"], b["offsets"],
                        b["row_of_slot"], b["src_of_row"], b["route_ws"], b["route_ws"].numel(), stream)
            L.moe_permute(sh, x, b["row_of_slot"], b["x_perm"], stream)
            L.moe_ep_send_plan(sh, ep, b["counts"], b["offsets"], b["send_counts"], b["send_offsets"], stream)
        L.moe_ep_exchange_counts_loopback(ep, el, [b["send_counts"] for b in self.src],
                                          [r["recv_counts"] for r in self.dst], stream)
        for r in self.dst:
            L.moe_ep_recv_plan(ep, el, self.rows_cap, r["recv_counts"], r["local_counts"], r["local_offsets"],
                               r["recv_offsets"], r["regroup_row"], stream)
        self._exchange("x_perm", "gx", False, stream)
        dsh = self.dst_shape()
        for i, r in enumerate(self.dst):
            sl = slice(i * el, (i + 1) * el)
            L.moe_grouped_gemm_fwd(dsh, r["gx"], w_gu[sl], w_down[sl], r["local_offsets"], r["h"], r["a"], r["gy"],
                                   r["fwd_ws"], r["fwd_ws"].numel(), stream)
        self._exchange("y_perm", "gy", True, stream)
        outs = []
        for s, T in enumerate(self.T):
            b = self.src[s]
            L.moe_unpermute_combine(self.src_shape(T), b["y_perm"], b["topk_w"], b["row_of_slot"], b["out"], stream)
            outs.append(b["out"][:T])
        return outs

    def backward(self, douts, w_gu, w_down, dw_gu, dw_down, stream=None):
        """Backward from the buffers of the last forward; dw_gu / dw_down hold
        all E experts and accumulate. Returns per-source dict of dx, dlogits,
        dtopk_w."""
        ep, el = self.ep, self.e_local
        for s, T in enumerate(self.T):
            b = self.src[s]
            sh = self.src_shape(T)
            L.moe_unpermute_combine_bwd(sh, douts[s], b["y_perm"], b["topk_w"], b["row_of_slot"], b["dy"],
                                        b["dtopk_w"], stream)
            L.moe_route_bwd(sh, b["dtopk_w"], b["logits"], b["topk_idx"], b["topk_w"], None, None, b["dlogits"], None,
                            None, b["route_ws"], b["route_ws"].numel(), stream)
        self._exchange("dy", "gy", False, stream)
        dsh = self.dst_shape()
        for i, r in enumerate(self.dst):
            sl = slice(i * el, (i + 1) * el)
            L.moe_grouped_gemm_bwd(dsh, r["gy"], r["gx"], r["h"], r["a"], w_gu[sl], w_down[sl], r["local_offsets"],
                                   r["gdx"], dw_gu[sl], dw_down[sl], r["bwd_ws"], r["bwd_ws"].numel(), stream)
        self._exchange("dx_perm", "gdx", True, stream)
        res = []
        for s, T in enumerate(self.T):
            b = self.src[s]
            L.moe_permute_bwd(self.src_shape(T), b["dx_perm"], b["row_of_slot"], None, b["dx"], stream)
            res.append(dict(dx=b["dx"][:T], dlogits=b["dlogits"][:T], dtopk_w=b["dtopk_w"][:T]))
        return res
