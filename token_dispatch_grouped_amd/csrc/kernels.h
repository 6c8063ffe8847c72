// Internal launch interface between the C ABI (moe_abi.cpp) and the HIP
// kernels. Every launcher enqueues on `stream`, makes no launch with an empty
// grid, and returns the HIP error of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "validate.h"

namespace moe {

// Geometry of the route pass: tokens per workgroup of the top-k kernel. The
// per-workgroup expert histograms ([nblk, E] int32) live in the route
// workspace.
constexpr int kRouteTokensPerBlock = kRouteTokens;
// Router weight-gradient partial sums: at most this many token chunks.
constexpr int kRouterMaxChunks = kRouterChunksMax;

inline int64_t route_blocks(int64_t T) { return (T + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock; }
inline int64_t router_chunk_tokens(int64_t T) {
  int64_t c = (T + kRouterMaxChunks - 1) / kRouterMaxChunks;
  return c < 256 ? 256 : c;
}
inline int64_t router_chunks(int64_t T) {
  int64_t c = router_chunk_tokens(T);
  return (T + c - 1) / c;
}

// Per-kernel timing hook (profiler in moe_abi.cpp). Brackets a launch with
// events when enabled; the pair joins the timer's records once both are
// recorded.
struct LaunchScope {
  LaunchScope(const char *name, hipStream_t s);
  ~LaunchScope();
  const char *name_;
  hipStream_t stream_;
  hipEvent_t start_, end_;
};

// ----- routing -----
hipError_t launch_router_logits(const void *x, const void *w_router, const float *bias, float *logits,
                                int64_t T, int d, int E, bool bf16, hipStream_t s);
hipError_t launch_route(const float *logits, int32_t *topk_idx, float *topk_w, int32_t *counts,
                        int32_t *offsets, int32_t *row_of_slot, int32_t *src_of_row, int32_t *blk_cnt,
                        int64_t T, int E, int k, bool renorm, hipStream_t s);
// Device address of the current GPU's static routing scratch
// (kRouteScratchBytes), looked up once per device.
hipError_t route_scratch(int32_t **out);
hipError_t launch_route_bwd(const float *dtopk_w, const float *logits, const int32_t *topk_idx,
                            const float *topk_w, float *dlogits, int64_t T, int E, int k, bool renorm,
                            bool accumulate, hipStream_t s);
hipError_t launch_router_bwd(const float *dlogits, const void *x, const void *w_router, float *dx_router,
                             float *dw_router, float *partial, int64_t T, int d, int E, bool bf16,
                             hipStream_t s);

// ----- data movement -----
hipError_t launch_permute(const void *x, const int32_t *row_of_slot, void *x_perm, int64_t T, int d,
                          int k, bool bf16, hipStream_t s);
hipError_t launch_combine(const void *y, const float *topk_w, const int32_t *row_of_slot, void *out,
                          int64_t T, int d, int k, bool bf16, hipStream_t s);
hipError_t launch_combine_bwd(const void *dout, const void *y, const float *topk_w,
                              const int32_t *row_of_slot, void *dy, float *dtopk_w, int64_t T, int d,
                              int k, bool bf16, hipStream_t s);
hipError_t launch_permute_bwd(const void *dx_perm, const int32_t *row_of_slot, const float *dx_extra,
                              void *dx, int64_t T, int d, int k, bool bf16, hipStream_t s);

// ----- grouped GEMMs -----
struct GroupedFfnArgs {
  const void *x_perm;   // [R, d]
  const void *w_gu;     // [E, 2F, d]
  const void *w_down;   // [E, d, F]
  const int32_t *offsets;  // [E+1]
  void *h;              // [R, 2F]
  void *a;              // [R, F]
  void *y;              // [R, d]
  // backward
  const void *dy;       // [R, d]
  void *dh;             // [R, 2F] (workspace)
  int32_t *order;       // [E] experts by descending row count (workspace)
  void *dx_perm;        // [R, d]
  float *dw_gu;         // [E, 2F, d]
  float *dw_down;       // [E, d, F]
  int64_t R;
  int d, E, F;
};
hipError_t launch_ffn_fwd_bf16(const GroupedFfnArgs &a, hipStream_t s);
hipError_t launch_ffn_bwd_bf16(const GroupedFfnArgs &a, hipStream_t s);
hipError_t launch_ffn_fwd_f32(const GroupedFfnArgs &a, hipStream_t s);
// Gate/up product + SwiGLU alone (h and a from x_perm), as in the forward;
// used to recompute the activations at the start of a backward.
hipError_t launch_ffn_recompute_bf16(const GroupedFfnArgs &a, hipStream_t s);
hipError_t launch_ffn_recompute_f32(const GroupedFfnArgs &a, hipStream_t s);
hipError_t launch_ffn_bwd_f32(const GroupedFfnArgs &a, hipStream_t s);

// Fused AdamW step (optim.hip). Scalars are prepared on the host: decay =
// 1 - lr*wd, step_size = lr / (1 - b1^t), bc2_sqrt = sqrt(1 - b2^t).
struct AdamwLaunch {
  float *theta, *grad, *m, *v;
  void *lowp;  // bf16 copy of theta, or NULL
  int64_t n;
  float b1, b2, decay, step_size, bc2_sqrt, eps, scale;
  bool zero_grad;
};
hipError_t launch_adamw(const AdamwLaunch &a, hipStream_t s);

// Auxiliary losses and routing metrics (aux.hip); partial: the route
// workspace, at least route_aux bytes.
hipError_t launch_aux_loss(const float *logits, const int32_t *counts, float *losses, float *metrics, float *dlogits,
                           float *partial, int64_t T, int E, int k, float alpha, float beta, bool accumulate,
                           hipStream_t s);

// ----- expert-parallel exchange (ep.hip) -----
struct EpPtrs {
  void *p[kEpMaxRanks];
};
struct EpCaps {
  int64_t n[kEpMaxRanks];
};
hipError_t launch_ep_send_plan(const int32_t *counts, const int32_t *offsets, int32_t *send_counts,
                               int32_t *send_offsets, int ep, int e_local, bool empty, hipStream_t s);
hipError_t launch_ep_recv_plan(const int32_t *recv_counts, int32_t *local_counts, int32_t *local_offsets,
                               int32_t *recv_offsets, int32_t *regroup_row, int64_t rows_cap, int ep, int e_local,
                               hipStream_t s);
hipError_t launch_ep_regroup(const void *src, void *dst, const int32_t *regroup_row, const int32_t *total,
                             int64_t rows_cap, int d, bool bf16, bool reverse, hipStream_t s);
hipError_t launch_ep_exchange_counts(const EpPtrs &send_counts, const EpPtrs &recv_counts, int ep, int e_local,
                                     hipStream_t s);
hipError_t launch_ep_exchange_rows(void *src, const int32_t *send_off, int64_t src_cap, const EpPtrs &dst,
                                   const EpPtrs &recv_off, const EpPtrs &regroup, const EpCaps &dst_cap, int source,
                                   int ep, int d, bool bf16, bool reverse, hipStream_t s);

// Attainable-peak probes (peak.hip): a bf16 MFMA loop on `cus` compute
// units and a plain device copy.
int peak_mfma_threads(int cus);
double peak_mfma_flops(int cus, int iters);
hipError_t launch_peak_mfma(float *out, int cus, int iters, hipStream_t s);
hipError_t launch_peak_copy(const void *src, void *dst, int64_t bytes, hipStream_t s);

}  // namespace moe
