"""Helpers for comparing the HIP path with the oracle (imported by tests,
the smoke check and the bench's CPU-baseline leg; not a test module)."""
from __future__ import annotations

import numpy as np

from workloads import BF16, F32, bf16_bits_to_f32, to_f64

# Parity bars: max|gpu - ref| / max|ref| per output tensor.
TOL = {BF16: 2e-2, F32: 1e-4}
# Routing weights and their gradients are computed in fp32 whatever the layer
# dtype is, so they take the fp32 bar.
TOL_ROUTING = 1e-4


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def to_host64(t) -> np.ndarray:
    """Device tensor (bf16/fp32/int) -> float64 numpy (exact widening)."""
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if gpu.size == 0:
        return 0.0
    if not np.all(np.isfinite(gpu)):
        return float("inf")
    m = float(np.max(np.abs(ref)))
    d = float(np.max(np.abs(gpu - ref)))
    if m == 0.0:
        return 0.0 if d == 0.0 else float("inf")
    return d / m


def assert_close(name: str, gpu, ref, tol: float):
    e = rel_err(gpu, ref)
    assert e <= tol, f"{name}: max|gpu-ref|/max|ref| = {e:.3e} > {tol:.1e}"
    return e


def f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return to_f64(a, dtype)


__all__ = ["TOL", "TOL_ROUTING", "to_device", "to_host64", "rel_err", "assert_close", "f64", "BF16", "F32"]
