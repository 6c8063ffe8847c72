"""ctypes binding of ``libmoe_mi355x.so`` (see ``include/moe.h``).

Argument marshalling only: every function here has the name of the C entry
point it calls, turns tensors into device pointers and the current torch
stream into a ``hipStream_t``, and raises :class:`MoeError` on a non-OK
status. No step of the layer is computed in Python, and there is no CPU
fallback: if the library has not been built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_MISALIGNED = 4
MOE_ERR_HIP = 5

MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_FLAG_RENORM = 1
MOE_FLAG_RECOMPUTE = 2
MOE_FLAG_ACCUMULATE_DLOGITS = 4
MOE_AUX_ACCUMULATE = 1
MOE_METRIC_IMBALANCE, MOE_METRIC_EMPTY_EXPERTS, MOE_METRIC_COUNT_CV, MOE_METRIC_ENTROPY, MOE_METRIC_MAX_PROB = range(5)
MOE_METRIC_SCALARS = 5


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({detail})")


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("F", ctypes.c_int32), ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


_P = ctypes.c_void_p
class moe_adamw_config(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("grad_scale", ctypes.c_float),
                ("step", ctypes.c_int64), ("flags", ctypes.c_uint32)]


MOE_ADAMW_ZERO_GRAD = 1


class moe_aux_config(ctypes.Structure):
    _fields_ = [("balance_coef", ctypes.c_float), ("z_coef", ctypes.c_float), ("flags", ctypes.c_uint32)]

_S = ctypes.POINTER(moe_shape)
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "moe_workspace_size": (ctypes.c_int, [_S, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
    "moe_route": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_noalloc": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_permute": (ctypes.c_int, [_S, _P, _P, _P, _P]),
    "moe_grouped_gemm_fwd": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_unpermute_combine": (ctypes.c_int, [_S, _P, _P, _P, _P, _P]),
    "moe_unpermute_combine_bwd": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P]),
    "moe_route_bwd": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_grouped_gemm_bwd": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute_bwd": (ctypes.c_int, [_S, _P, _P, _P, _P, _P]),
    "moe_aux_loss": (ctypes.c_int, [_S, _P, _P, ctypes.POINTER(moe_aux_config), _P, _P, _P, _P, _SZ, _P]),
    "moe_adamw_step": (ctypes.c_int, [ctypes.POINTER(moe_adamw_config), ctypes.c_int64, _P, _P, _P, _P, _P, _P]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_profiler_enable": (ctypes.c_int, [ctypes.c_int]),
    "moe_profiler_reset": (ctypes.c_int, []),
    "moe_profiler_count": (ctypes.c_int, []),
    "moe_profiler_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                         ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]),
    "moe_version": (ctypes.c_char_p, []),
    "moe_ep_send_plan": (ctypes.c_int, [_S, ctypes.c_int32, _P, _P, _P, _P, _P]),
    "moe_ep_recv_plan": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, _P, _P, _P, _P, _P, _P]),
    "moe_ep_regroup": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _P, _P, _P, _P,
                                      ctypes.c_int32, _P]),
    "moe_ep_exchange_counts_loopback": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "moe_ep_exchange_loopback": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P, _P,
                                                _P, ctypes.c_int32, _P]),
    # include/moe_peak.h
    "moe_peak_mfma": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.POINTER(ctypes.c_double), _P]),
    "moe_peak_mfma_size": (ctypes.c_int64, []),
    "moe_peak_copy": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P]),
}

_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build the HIP library first "
                           "(python -m token_dispatch_grouped_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_names():
    return list(_SIGNATURES)


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def ptr(t) -> Optional[int]:
    """Device pointer of a tensor (or an int address, or None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def current_stream() -> Optional[int]:
    import torch
    if not torch.cuda.is_available():
        return None
    return torch.cuda.current_stream().cuda_stream


def make_shape(T: int, d: int, E: int, k: int, F: int, dtype: int, flags: int = 0) -> moe_shape:
    return moe_shape(int(T), int(d), int(E), int(k), int(F), int(dtype), int(flags))


def _check(status: int, where: str):
    if status != MOE_OK:
        lib = load()
        raise MoeError(status, where, lib.moe_last_error().decode() or lib.moe_status_string(status).decode())


def _stream(stream):
    return current_stream() if stream is None else stream


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def moe_workspace_size(shape: moe_shape):
    lib = load()
    a, b, c = _SZ(), _SZ(), _SZ()
    _check(lib.moe_workspace_size(ctypes.byref(shape), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
           "moe_workspace_size")
    return a.value, b.value, c.value


def moe_route(shape, x, w_router, bias, logits, topk_idx, topk_w, counts, offsets, row_of_slot, src_of_row,
              ws, ws_bytes, stream=None):
    lib = load()
    _check(lib.moe_route(ctypes.byref(shape), ptr(x), ptr(w_router), ptr(bias), ptr(logits), ptr(topk_idx),
                         ptr(topk_w), ptr(counts), ptr(offsets), ptr(row_of_slot), ptr(src_of_row), ptr(ws),
                         int(ws_bytes), _stream(stream)), "moe_route")


def moe_route_noalloc(shape, x, w_router, bias, logits, topk_idx, topk_w, counts, offsets, row_of_slot,
                      src_of_row, stream=None):
    lib = load()
    _check(lib.moe_route_noalloc(ctypes.byref(shape), ptr(x), ptr(w_router), ptr(bias), ptr(logits), ptr(topk_idx),
                                 ptr(topk_w), ptr(counts), ptr(offsets), ptr(row_of_slot), ptr(src_of_row),
                                 _stream(stream)), "moe_route_noalloc")


def moe_permute(shape, x, row_of_slot, x_perm, stream=None):
    lib = load()
    _check(lib.moe_permute(ctypes.byref(shape), ptr(x), ptr(row_of_slot), ptr(x_perm), _stream(stream)),
           "moe_permute")


def moe_grouped_gemm_fwd(shape, x_perm, w_gu, w_down, offsets, h, a, y, ws, ws_bytes, stream=None):
    lib = load()
    _check(lib.moe_grouped_gemm_fwd(ctypes.byref(shape), ptr(x_perm), ptr(w_gu), ptr(w_down), ptr(offsets), ptr(h),
                                    ptr(a), ptr(y), ptr(ws), int(ws_bytes), _stream(stream)), "moe_grouped_gemm_fwd")


def moe_unpermute_combine(shape, y, topk_w, row_of_slot, out, stream=None):
    lib = load()
    _check(lib.moe_unpermute_combine(ctypes.byref(shape), ptr(y), ptr(topk_w), ptr(row_of_slot), ptr(out),
                                     _stream(stream)), "moe_unpermute_combine")


def moe_unpermute_combine_bwd(shape, dout, y, topk_w, row_of_slot, dy, dtopk_w, stream=None):
    lib = load()
    _check(lib.moe_unpermute_combine_bwd(ctypes.byref(shape), ptr(dout), ptr(y), ptr(topk_w), ptr(row_of_slot),
                                         ptr(dy), ptr(dtopk_w), _stream(stream)), "moe_unpermute_combine_bwd")


def moe_route_bwd(shape, dtopk_w, logits, topk_idx, topk_w, x, w_router, dlogits, dx_router, dw_router, ws,
                  ws_bytes, stream=None):
    lib = load()
    _check(lib.moe_route_bwd(ctypes.byref(shape), ptr(dtopk_w), ptr(logits), ptr(topk_idx), ptr(topk_w), ptr(x),
                             ptr(w_router), ptr(dlogits), ptr(dx_router), ptr(dw_router), ptr(ws), int(ws_bytes),
                             _stream(stream)), "moe_route_bwd")


def moe_grouped_gemm_bwd(shape, dy, x_perm, h, a, w_gu, w_down, offsets, dx_perm, dw_gu, dw_down, ws, ws_bytes,
                         stream=None):
    lib = load()
    _check(lib.moe_grouped_gemm_bwd(ctypes.byref(shape), ptr(dy), ptr(x_perm), ptr(h), ptr(a), ptr(w_gu),
                                    ptr(w_down), ptr(offsets), ptr(dx_perm), ptr(dw_gu), ptr(dw_down), ptr(ws),
                                    int(ws_bytes), _stream(stream)), "moe_grouped_gemm_bwd")


def moe_permute_bwd(shape, dx_perm, row_of_slot, dx_extra, dx, stream=None):
    lib = load()
    _check(lib.moe_permute_bwd(ctypes.byref(shape), ptr(dx_perm), ptr(row_of_slot), ptr(dx_extra), ptr(dx),
                               _stream(stream)), "moe_permute_bwd")


def make_aux_config(balance_coef: float, z_coef: float, accumulate: bool = False) -> moe_aux_config:
    return moe_aux_config(float(balance_coef), float(z_coef), MOE_AUX_ACCUMULATE if accumulate else 0)


def moe_aux_loss(shape, logits, counts, cfg, losses, metrics, dlogits, ws, ws_bytes, stream=None):
    lib = load()
    _check(lib.moe_aux_loss(ctypes.byref(shape), ptr(logits), ptr(counts), ctypes.byref(cfg), ptr(losses),
                            ptr(metrics), ptr(dlogits), ptr(ws), int(ws_bytes), _stream(stream)), "moe_aux_loss")


def make_adamw_config(lr: float, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                      weight_decay: float = 0.01, grad_scale: float = 1.0, step: int = 1,
                      zero_grad: bool = False) -> moe_adamw_config:
    return moe_adamw_config(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
                            float(grad_scale), int(step), MOE_ADAMW_ZERO_GRAD if zero_grad else 0)


def moe_adamw_step(cfg, n, param, grad, exp_avg, exp_avg_sq, param_bf16=None, stream=None):
    lib = load()
    _check(lib.moe_adamw_step(ctypes.byref(cfg), int(n), ptr(param), ptr(grad), ptr(exp_avg), ptr(exp_avg_sq),
                              ptr(param_bf16), _stream(stream)), "moe_adamw_step")


MOE_EP_MAX_RANKS = 8


def _ptr_array(items):
    """Host array of device pointers (None -> NULL) for the per-rank arguments."""
    arr = (ctypes.c_void_p * len(items))(*[ptr(t) for t in items])
    return ctypes.cast(arr, ctypes.c_void_p), arr


def _i64_array(vals):
    arr = (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])
    return ctypes.cast(arr, ctypes.c_void_p), arr


def moe_ep_send_plan(shape, ep, counts, offsets, send_counts, send_offsets, stream=None):
    _check(load().moe_ep_send_plan(ctypes.byref(shape), int(ep), ptr(counts), ptr(offsets), ptr(send_counts),
                                   ptr(send_offsets), _stream(stream)), "moe_ep_send_plan")


def moe_ep_recv_plan(ep, e_local, rows_cap, recv_counts, local_counts, local_offsets, recv_offsets, regroup_row,
                     stream=None):
    _check(load().moe_ep_recv_plan(int(ep), int(e_local), int(rows_cap), ptr(recv_counts), ptr(local_counts),
                                   ptr(local_offsets), ptr(recv_offsets), ptr(regroup_row), _stream(stream)),
           "moe_ep_recv_plan")


def moe_ep_regroup(d, dtype, rows_cap, ep, recv_offsets, regroup_row, src, dst, reverse=False, stream=None):
    _check(load().moe_ep_regroup(int(d), int(dtype), int(rows_cap), int(ep), ptr(recv_offsets), ptr(regroup_row),
                                 ptr(src), ptr(dst), 1 if reverse else 0, _stream(stream)), "moe_ep_regroup")


def moe_ep_exchange_counts_loopback(ep, e_local, send_counts, recv_counts, stream=None):
    sp, _a = _ptr_array(send_counts)
    rp, _b = _ptr_array(recv_counts)
    _check(load().moe_ep_exchange_counts_loopback(int(ep), int(e_local), sp, rp, _stream(stream)),
           "moe_ep_exchange_counts_loopback")


def moe_ep_exchange_loopback(ep, d, dtype, send_bufs, send_caps, send_offsets, recv_bufs, recv_caps, recv_offsets,
                             regroup_rows=None, reverse=False, stream=None):
    a = [_ptr_array(send_bufs), _i64_array(send_caps), _ptr_array(send_offsets), _ptr_array(recv_bufs),
         _i64_array(recv_caps), _ptr_array(recv_offsets)]
    rg = _ptr_array(regroup_rows) if regroup_rows is not None else (None, None)
    _check(load().moe_ep_exchange_loopback(int(ep), int(d), int(dtype), *[x[0] for x in a], rg[0],
                                           1 if reverse else 0, _stream(stream)), "moe_ep_exchange_loopback")


def moe_peak_mfma_size() -> int:
    return int(load().moe_peak_mfma_size())


def moe_peak_mfma(out, iters: int, stream=None) -> float:
    """Launch the bf16 MFMA loop; returns the FLOPs of the launch."""
    fl = ctypes.c_double()
    _check(load().moe_peak_mfma(ptr(out), int(iters), ctypes.byref(fl), _stream(stream)), "moe_peak_mfma")
    return fl.value


def moe_peak_copy(src, dst, nbytes: int, stream=None):
    _check(load().moe_peak_copy(ptr(src), ptr(dst), int(nbytes), _stream(stream)), "moe_peak_copy")


def moe_status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def moe_last_error() -> str:
    return load().moe_last_error().decode()


def moe_version() -> str:
    return load().moe_version().decode()


def moe_profiler_enable(on: bool):
    _check(load().moe_profiler_enable(1 if on else 0), "moe_profiler_enable")


def moe_profiler_reset():
    _check(load().moe_profiler_reset(), "moe_profiler_reset")


def moe_profiler_read_all():
    """{kernel name: (launches, total ms)} since the last reset."""
    lib = load()
    out = {}
    for i in range(lib.moe_profiler_count()):
        name = ctypes.c_char_p()
        n = ctypes.c_int64()
        ms = ctypes.c_double()
        _check(lib.moe_profiler_read(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms)), "moe_profiler_read")
        out[name.value.decode()] = (n.value, ms.value)
    return out
