"""Buffer management and call sequence of one MoE layer over the C ABI.

PyTorch is used here only to allocate device memory and to provide the
stream: every step of the forward and backward runs in the library's HIP
kernels, in this order

  forward : moe_route -> moe_permute -> moe_grouped_gemm_fwd -> moe_unpermute_combine
  backward: moe_unpermute_combine_bwd -> moe_route_bwd -> moe_grouped_gemm_bwd -> moe_permute_bwd

All activation buffers and workspaces are allocated once for the largest
microbatch (``T_max``) and reused for any smaller one: microbatches of
changing size, the empty one included, run on the same buffers ("buffer
capacity transitions"). Weight gradients are fp32 and accumulate across
calls; the caller zeroes them once.

With ``recompute=True`` (MOE_FLAG_RECOMPUTE) the layer keeps no h or a
buffers: the forward holds a in its workspace only and the backward
recomputes h and a from x_perm. The same layer object also serves a
forward with no backward after it (no-grad execution).

With ``aux=(balance_coef, z_coef)`` the forward also computes the auxiliary
losses (load balancing, router z-loss) and the routing metrics into
``aux_losses`` / ``metrics``, and the backward adds the losses' gradient to
dlogits before the routing-weight gradient (MOE_FLAG_ACCUMULATE_DLOGITS), so
a router trains on both.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import _lib as L


def torch_dtype(moe_dtype: int):
    return torch.bfloat16 if moe_dtype == L.MOE_DTYPE_BF16 else torch.float32


@dataclasses.dataclass
class Saved:
    """Views of the forward's saved tensors for one microbatch of T tokens."""
    T: int
    logits: torch.Tensor
    topk_idx: torch.Tensor
    topk_w: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    row_of_slot: torch.Tensor
    src_of_row: torch.Tensor
    x_perm: torch.Tensor
    h: Optional[torch.Tensor]  # None under recompute
    a: Optional[torch.Tensor]  # None under recompute
    y: torch.Tensor
    out: torch.Tensor


class MoeLayer:
    def __init__(self, T_max: int, d: int, E: int, k: int, F: int, dtype: int = L.MOE_DTYPE_BF16,
                 renorm: bool = False, router: bool = False, recompute: bool = False, aux=None,
                 device: str = "cuda"):
        self.T_max, self.d, self.E, self.k, self.F = T_max, d, E, k, F
        self.dtype = dtype
        self.recompute = recompute
        self.aux = None if aux is None else (float(aux[0]), float(aux[1]))
        self.flags = ((L.MOE_FLAG_RENORM if renorm else 0) | (L.MOE_FLAG_RECOMPUTE if recompute else 0)
                      | (L.MOE_FLAG_ACCUMULATE_DLOGITS if aux is not None else 0))
        self.router = router
        dev = torch.device(device)
        td = torch_dtype(dtype)
        R = T_max * k
        shape = self.shape(T_max)
        self.route_ws_bytes, self.fwd_ws_bytes, self.bwd_ws_bytes = L.moe_workspace_size(shape)
        u8 = torch.uint8
        self.route_ws = torch.empty(max(self.route_ws_bytes, 256), dtype=u8, device=dev)
        self.fwd_ws = torch.empty(max(self.fwd_ws_bytes, 256), dtype=u8, device=dev)
        self.bwd_ws = torch.empty(max(self.bwd_ws_bytes, 256), dtype=u8, device=dev)
        f32, i32 = torch.float32, torch.int32
        self.logits = torch.empty(T_max, E, dtype=f32, device=dev)
        self.topk_idx = torch.empty(T_max, k, dtype=i32, device=dev)
        self.topk_w = torch.empty(T_max, k, dtype=f32, device=dev)
        self.counts = torch.zeros(E, dtype=i32, device=dev)
        self.offsets = torch.zeros(E + 1, dtype=i32, device=dev)
        self.row_of_slot = torch.empty(T_max, k, dtype=i32, device=dev)
        self.src_of_row = torch.empty(R, dtype=i32, device=dev)
        self.x_perm = torch.empty(R, d, dtype=td, device=dev)
        self.h = None if recompute else torch.empty(R, 2 * F, dtype=td, device=dev)
        self.a = None if recompute else torch.empty(R, F, dtype=td, device=dev)
        self.y = torch.empty(R, d, dtype=td, device=dev)
        self.out = torch.empty(T_max, d, dtype=td, device=dev)
        # backward
        self.dy = torch.empty(R, d, dtype=td, device=dev)
        self.dtopk_w = torch.empty(T_max, k, dtype=f32, device=dev)
        self.dlogits = torch.empty(T_max, E, dtype=f32, device=dev)
        self.dx_perm = torch.empty(R, d, dtype=td, device=dev)
        self.dx = torch.empty(T_max, d, dtype=td, device=dev)
        self.dx_router = torch.empty(T_max, d, dtype=f32, device=dev) if router else None
        # auxiliary losses (L_bal, L_z) and routing metrics of the last forward
        self.aux_losses = torch.zeros(2, dtype=f32, device=dev) if aux is not None else None
        self.metrics = torch.zeros(L.MOE_METRIC_SCALARS + 2 * E, dtype=f32, device=dev) if aux is not None else None

    def shape(self, T: int) -> L.moe_shape:
        return L.make_shape(T, self.d, self.E, self.k, self.F, self.dtype, self.flags)

    def saved(self, T: int) -> Saved:
        R = T * self.k
        return Saved(T, self.logits[:T], self.topk_idx[:T], self.topk_w[:T], self.counts, self.offsets,
                     self.row_of_slot[:T], self.src_of_row[:R], self.x_perm[:R],
                     None if self.h is None else self.h[:R], None if self.a is None else self.a[:R],
                     self.y[:R], self.out[:T])

    # ------------------------------------------------------------------
    def route(self, T: int, x=None, logits=None, w_router=None, bias=None, stream=None):
        s = self.shape(T)
        if w_router is None and logits is not None and T:
            self.logits[:T].copy_(logits)
        L.moe_route(s, x if w_router is not None else None, w_router, bias, self.logits, self.topk_idx, self.topk_w,
                    self.counts, self.offsets, self.row_of_slot, self.src_of_row, self.route_ws,
                    self.route_ws.numel(), stream)

    def forward(self, T: int, x, w_gu, w_down, logits=None, w_router=None, bias=None, stream=None) -> Saved:
        """One forward. ``logits`` (fp32 [T,E]) are copied into the layer's
        logits buffer unless a router weight is given."""
        s = self.shape(T)
        self.route(T, x=x, logits=logits, w_router=w_router, bias=bias, stream=stream)
        if self.aux is not None:
            L.moe_aux_loss(s, self.logits, self.counts, L.make_aux_config(*self.aux), self.aux_losses, self.metrics,
                           None, self.route_ws, self.route_ws.numel(), stream)
        L.moe_permute(s, x, self.row_of_slot, self.x_perm, stream)
        L.moe_grouped_gemm_fwd(s, self.x_perm, w_gu, w_down, self.offsets, self.h, self.a, self.y, self.fwd_ws,
                               self.fwd_ws.numel(), stream)
        L.moe_unpermute_combine(s, self.y, self.topk_w, self.row_of_slot, self.out, stream)
        return self.saved(T)

    def backward(self, T: int, dout, w_gu, w_down, dw_gu, dw_down, x=None, w_router=None, dw_router=None,
                 stream=None):
        """One backward from the buffers of the last forward; dw_* accumulate."""
        s = self.shape(T)
        L.moe_unpermute_combine_bwd(s, dout, self.y, self.topk_w, self.row_of_slot, self.dy, self.dtopk_w, stream)
        use_router = w_router is not None
        if self.aux is not None:  # aux gradient first; moe_route_bwd then adds to it
            L.moe_aux_loss(s, self.logits, self.counts, L.make_aux_config(*self.aux), None, None, self.dlogits,
                           self.route_ws, self.route_ws.numel(), stream)
        L.moe_route_bwd(s, self.dtopk_w, self.logits, self.topk_idx, self.topk_w, x if use_router else None,
                        w_router, self.dlogits, self.dx_router if use_router else None,
                        dw_router if use_router else None, self.route_ws, self.route_ws.numel(), stream)
        L.moe_grouped_gemm_bwd(s, self.dy, self.x_perm, self.h, self.a, w_gu, w_down, self.offsets, self.dx_perm,
                               dw_gu, dw_down, self.bwd_ws, self.bwd_ws.numel(), stream)
        L.moe_permute_bwd(s, self.dx_perm, self.row_of_slot, self.dx_router if use_router else None, self.dx,
                          stream)
        R = T * self.k
        return dict(dy=self.dy[:R], dtopk_w=self.dtopk_w[:T], dlogits=self.dlogits[:T], dx_perm=self.dx_perm[:R],
                    dx=self.dx[:T], dh=self.dh_view(T),
                    dx_router=self.dx_router[:T] if use_router else None)

    def fwd_a_view(self, T: int) -> torch.Tensor:
        """Under recompute: a of the last forward, read from the forward
        workspace (valid until the next forward)."""
        assert self.recompute, "a lives in the forward workspace only under recompute"
        R = T * self.k
        td = torch_dtype(self.dtype)
        es = 2 if td == torch.bfloat16 else 4
        return self.fwd_ws[: R * self.F * es].view(td).view(R, self.F)

    def dh_view(self, T: int) -> torch.Tensor:
        """dH of the last backward, read from the backward workspace."""
        R = T * self.k
        td = torch_dtype(self.dtype)
        es = 2 if td == torch.bfloat16 else 4
        return self.bwd_ws[: R * 2 * self.F * es].view(td).view(R, 2 * self.F)
