"""AdamW for the expert weights over the C ABI (``moe_adamw_step``).

Keeps fp32 master weights and both moments for each expert weight tensor
(w_gu [E,2F,d] and w_down [E,d,F]); each ``step`` runs one fused pass per
tensor that updates master and moments, writes the bf16 working copy the
grouped GEMMs read (in place, in the layer's weight tensor) and zeroes the
fp32 gradient the backward accumulated into. PyTorch only allocates.
"""
from __future__ import annotations

from typing import List, Sequence

import torch

from . import _lib as L


class ExpertAdamW:
    def __init__(self, weights: Sequence[torch.Tensor], lr: float, betas=(0.9, 0.999), eps: float = 1e-8,
                 weight_decay: float = 0.01):
        """``weights``: the working tensors the layer reads. A bf16 weight
        gets an fp32 master that starts as its exact widening; an fp32
        weight is its own master (updated in place)."""
        self.weights: List[torch.Tensor] = list(weights)
        for w in self.weights:
            if not w.is_contiguous() or w.dtype not in (torch.bfloat16, torch.float32):
                raise ValueError("expert weights must be contiguous bf16 or fp32 tensors")
        self.master = [w.detach().float().clone() if w.dtype == torch.bfloat16 else w for w in self.weights]
        self.exp_avg = [torch.zeros_like(m) for m in self.master]
        self.exp_avg_sq = [torch.zeros_like(m) for m in self.master]
        self.lr, self.betas, self.eps, self.weight_decay = lr, tuple(betas), eps, weight_decay
        self.t = 0

    def step(self, grads: Sequence[torch.Tensor], grad_scale: float = 1.0, zero_grad: bool = True, stream=None):
        """One update from fp32 gradients (same shapes as the weights)."""
        self.t += 1
        cfg = L.make_adamw_config(self.lr, self.betas[0], self.betas[1], self.eps, self.weight_decay, grad_scale,
                                  self.t, zero_grad)
        for w, mst, g, m, v in zip(self.weights, self.master, grads, self.exp_avg, self.exp_avg_sq):
            if g.dtype != torch.float32 or g.shape != mst.shape or not g.is_contiguous():
                raise ValueError("gradients must be contiguous fp32 tensors shaped like the weights")
            L.moe_adamw_step(cfg, mst.numel(), mst, g, m, v, w if w.dtype == torch.bfloat16 else None, stream)
