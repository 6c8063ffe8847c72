"""MI355X-native MoE token dispatch, grouped SwiGLU expert FFN and combine.

The compute lives in ``libmoe_mi355x.so`` (HIP kernels for gfx950 behind the
C ABI declared in ``include/moe.h``); this package is its Python binding.
"""
from ._lib import (  # noqa: F401
    MOE_DTYPE_BF16, MOE_DTYPE_F32, MOE_FLAG_RECOMPUTE, MOE_FLAG_RENORM, MOE_OK, MOE_ERR_HIP, MOE_ERR_INVALID_ARGUMENT,
    MOE_ERR_MISALIGNED, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MoeError, load, make_shape, moe_shape,
    moe_workspace_size, moe_route, moe_route_noalloc, moe_permute, moe_grouped_gemm_fwd, moe_unpermute_combine,
    moe_unpermute_combine_bwd, moe_route_bwd, moe_grouped_gemm_bwd, moe_permute_bwd, moe_status_string,
    moe_last_error, moe_version, moe_profiler_enable, moe_profiler_reset, moe_profiler_read_all,
    MOE_ADAMW_ZERO_GRAD, make_adamw_config, moe_adamw_config, moe_adamw_step,
    MOE_FLAG_ACCUMULATE_DLOGITS, MOE_AUX_ACCUMULATE, MOE_METRIC_IMBALANCE, MOE_METRIC_EMPTY_EXPERTS,
    MOE_METRIC_COUNT_CV, MOE_METRIC_ENTROPY, MOE_METRIC_MAX_PROB, MOE_METRIC_SCALARS, make_aux_config,
    moe_aux_config, moe_aux_loss, moe_peak_mfma, moe_peak_mfma_size, moe_peak_copy,
    MOE_EP_MAX_RANKS, moe_ep_send_plan, moe_ep_recv_plan, moe_ep_regroup, moe_ep_exchange_counts_loopback,
    moe_ep_exchange_loopback,
)

__all__ = [n for n in dir() if n.startswith(("moe_", "MOE_"))] + ["MoeError", "load", "make_shape",
                                                                  "make_adamw_config", "make_aux_config"]
