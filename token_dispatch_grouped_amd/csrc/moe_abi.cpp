// The C ABI of the MoE library: argument validation, workspace carving,
// kernel launches on the caller's stream, status codes, and the optional
// per-kernel event timer.
//
// Every entry point validates all of its arguments on the host before it
// launches anything (explicit errors for unsupported configurations: Support
// combined expert and data parallelism in TrainerRank, Current behavior and
// Desired behavior). An empty microbatch (T = 0) is a successful no-op, so
// uneven or empty work never needs special handling by the caller (same page,
// Desired behavior and Acceptance).
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "moe.h"
#include "moe_peak.h"
#include "kernels.h"
#include "validate.h"

namespace moe {

// A roctx range around each C-ABI call, so that a marker trace shows the
// calls above their kernels (rocprofv3 --marker-trace). Costs nothing
// measurable when no tool listens.
struct AbiRange {
  explicit AbiRange(const char *name) { roctxRangePushA(name); }
  ~AbiRange() { roctxRangePop(); }
};


static thread_local std::string g_last_error;

static moe_status report(moe_status st, const std::string &why) {
  g_last_error = why;
  return st;
}

static moe_status hip_status(hipError_t err, const char *where) {
  if (err == hipSuccess) return MOE_OK;
  std::string why = std::string(where) + ": " + hipGetErrorString(err);
  return report(MOE_ERR_HIP, why);
}

// ---------------------------------------------------------------------------
// event timer
// ---------------------------------------------------------------------------
struct ProfEntry {
  const char *name;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> live;  // recorded, not yet read
  int64_t launches = 0;
  double ms = 0.0;
};

// Process-wide; every member but `on` is used under `mu`, so launches on
// several threads (and reads beside them) may be timed together.
struct Profiler {
  std::atomic<bool> on{false};
  std::mutex mu;
  std::vector<ProfEntry> entries;
  std::vector<hipEvent_t> pool;

  hipEvent_t take() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  int slot(const char *name) {
    for (size_t i = 0; i < entries.size(); ++i)
      if (strcmp(entries[i].name, name) == 0) return (int)i;
    entries.push_back(ProfEntry{name, {}, 0, 0.0});
    return (int)entries.size() - 1;
  }
  // fold completed event pairs of entry i into its totals
  void drain(int i) {
    ProfEntry &en = entries[i];
    for (auto &pr : en.live) {
      float ms = 0.f;
      (void)hipEventSynchronize(pr.second);
      if (hipEventElapsedTime(&ms, pr.first, pr.second) == hipSuccess) en.ms += ms;
      en.launches += 1;
      pool.push_back(pr.first);
      pool.push_back(pr.second);
    }
    en.live.clear();
  }
};

static Profiler g_prof;

LaunchScope::LaunchScope(const char *name, hipStream_t s) : name_(name), stream_(s), start_(nullptr), end_(nullptr) {
  if (!g_prof.on.load(std::memory_order_relaxed)) return;
  {
    std::lock_guard<std::mutex> lock(g_prof.mu);
    start_ = g_prof.take();
    end_ = g_prof.take();
  }
  if (!start_ || !end_) {  // no events: this launch goes untimed
    std::lock_guard<std::mutex> lock(g_prof.mu);
    if (start_) g_prof.pool.push_back(start_);
    if (end_) g_prof.pool.push_back(end_);
    start_ = end_ = nullptr;
    return;
  }
  (void)hipEventRecord(start_, s);
}

// The pair is handed to the timer only now that both events are recorded,
// so a read never waits on an event that has not been recorded yet.
LaunchScope::~LaunchScope() {
  if (!end_) return;
  (void)hipEventRecord(end_, stream_);
  std::lock_guard<std::mutex> lock(g_prof.mu);
  g_prof.entries[g_prof.slot(name_)].live.push_back({start_, end_});
}

}  // namespace moe

using namespace moe;

static inline hipStream_t as_stream(moe_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

extern "C" {

const char *moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

const char *moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case MOE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char *moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_workspace_size(const moe_shape *shape, size_t *route_ws, size_t *gemm_fwd_ws,
                              size_t *gemm_bwd_ws) {
  std::string why;
  moe_status st = validate_shape(shape, &why);
  if (st != MOE_OK) return report(st, why);
  const WorkspaceLayout w = workspace_layout(*shape);
  if (route_ws) *route_ws = w.route_total;
  if (gemm_fwd_ws) *gemm_fwd_ws = w.gemm_fwd_total;
  if (gemm_bwd_ws) *gemm_bwd_ws = w.gemm_bwd_total;
  g_last_error.clear();
  return MOE_OK;
}

moe_status moe_route(const moe_shape *shape, const void *x, const void *w_router, const float *bias, float *logits,
                     int32_t *topk_idx, float *topk_w, int32_t *counts, int32_t *offsets, int32_t *row_of_slot,
                     int32_t *src_of_row, void *ws, size_t ws_bytes, moe_stream_t stream) {
  moe::AbiRange range("moe_route");
  std::string why;
  moe_status st = validate_shape(shape, &why);
  if (st != MOE_OK) return report(st, why);
  const moe_shape &s = *shape;
  if (s.T == 0) return MOE_OK;
  const bool router = w_router != nullptr;
  const PtrArg args[] = {
      {"x", x, router, !router},
      {"w_router", w_router, false, false},
      {"bias", bias, false, !router},
      {"logits", logits, true, false},
      {"topk_idx", topk_idx, true, false},
      {"topk_w", topk_w, true, false},
      {"counts", counts, true, false},
      {"offsets", offsets, true, false},
      {"row_of_slot", row_of_slot, true, false},
      {"src_of_row", src_of_row, true, false},
  };
  st = validate_ptrs(args, sizeof(args) / sizeof(args[0]), &why);
  if (st != MOE_OK) return report(st, why);
  const WorkspaceLayout w = workspace_layout(s);
  st = validate_workspace(ws, ws_bytes, w.route_total, &why);
  if (st != MOE_OK) return report(st, why);

  hipStream_t hs = as_stream(stream);
  const bool bf16 = s.dtype == MOE_DTYPE_BF16;
  if (router) {
    st = hip_status(launch_router_logits(x, w_router, bias, logits, s.T, s.d, s.E, bf16, hs), "router_logits");
    if (st != MOE_OK) return st;
  }
  int32_t *blk_cnt = reinterpret_cast<int32_t *>(ws);
  return hip_status(launch_route(logits, topk_idx, topk_w, counts, offsets, row_of_slot, src_of_row, blk_cnt, s.T,
                                 s.E, s.k, (s.flags & MOE_FLAG_RENORM) != 0, hs),
                    "route");
}

moe_status moe_route_noalloc(const moe_shape *shape, const void *x, const void *w_router, const float *bias,
                             float *logits, int32_t *topk_idx, float *topk_w, int32_t *counts, int32_t *offsets,
                             int32_t *row_of_slot, int32_t *src_of_row, moe_stream_t stream) {
  moe::AbiRange range("moe_route_noalloc");
  std::string why;
  moe_status st = validate_shape(shape, &why);
  if (st != MOE_OK) return report(st, why);
  const moe_shape &s = *shape;
  if (s.T == 0) return MOE_OK;
  const bool router = w_router != nullptr;
  const PtrArg args[] = {
      {"x", x, router, !router},
      {"w_router", w_router, false, false},
      {"bias", bias, false, !router},
      {"logits", logits, true, false},
      {"topk_idx", topk_idx, true, false},
      {"topk_w", topk_w, true, false},
      {"counts", counts, true, false},
      {"offsets", offsets, true, false},
      {"row_of_slot", row_of_slot, true, false},
      {"src_of_row", src_of_row, true, false},
  };
  st = validate_ptrs(args, sizeof(args) / sizeof(args[0]), &why);
  if (st != MOE_OK) return report(st, why);
  const WorkspaceLayout w = workspace_layout(s);
  if (w.route_blk_cnt > kRouteScratchBytes) {
    char buf[200];
    snprintf(buf, sizeof buf,
             "moe_route_noalloc: T=%lld, E=%d needs %zu bytes of routing scratch; the static scratch holds %zu "
             "(use moe_route with a workspace)",
             (long long)s.T, s.E, w.route_blk_cnt, kRouteScratchBytes);
    return report(MOE_ERR_UNSUPPORTED, buf);
  }
  int32_t *blk_cnt = nullptr;
  st = hip_status(route_scratch(&blk_cnt), "moe_route_noalloc (scratch address)");
  if (st != MOE_OK) return st;
  hipStream_t hs = as_stream(stream);
  const bool bf16 = s.dtype == MOE_DTYPE_BF16;
  if (router) {
    st = hip_status(launch_router_logits(x, w_router, bias, logits, s.T, s.d, s.E, bf16, hs), "router_logits");
    if (st != MOE_OK) return st;
  }
  return hip_status(launch_route(logits, topk_idx, topk_w, counts, offsets, row_of_slot, src_of_row, blk_cnt, s.T,
                                 s.E, s.k, (s.flags & MOE_FLAG_RENORM) != 0, hs),
                    "route");
}

moe_status moe_permute(const moe_shape *shape, const void *x, const int32_t *row_of_slot, void *x_perm,
                       moe_stream_t stream) {
  moe::AbiRange range("moe_permute");
  std::string why;
  moe_status st = validate_shape(shape, &why);
  if (st != MOE_OK) return report(st, why);
  const moe_shape &s = *shape;
  if (s.T == 0) return MOE_OK;
  const PtrArg args[] = {{"x", x, true, false}, {"row_of_slot", row_of_slot, true, false}, {"x_perm", x_perm, true, false}};
  st = validate_ptrs(args, 3, &why);
  if (st != MOE_OK) return report(st, why);
  return hip_status(launch_permute(x, row_of_slot, x_perm, s.T, s.d, s.k, s.dtype == MOE_DTYPE_BF16, as_stream(stream)),
                    "permute");
}

static GroupedFfnArgs ffn_args(const moe_shape &s) {
  GroupedFfnArgs a{};
  a.R = s.T * (int64_t)s.k;
  a.d = s.d;
  a.E = s.E;
  a.F = s.F;
  return a;
}

moe_status moe_grouped_gemm_fwd(const moe_shape *shape, const void *x_perm, const void *w_gu, const void *w_down,
                                const int32_t *offsets, void *h, void *a, void *y, void *ws, size_t ws_bytes,
                                moe_stream_t stream) {
  moe::AbiRange range("moe_grouped_gemm_fwd");
  std::string why;
  moe_status st = validate_shape(shape, &why);
  if (st != MOE_OK) return report(st, why);
  const moe_shape &s = *shape;
  if (s.T == 0) return MOE_OK;
  const bool rc = (s.flags & MOE_FLAG_RECOMPUTE) != 0;
  const PtrArg args[] = {{"x_perm", x_perm, true, false}, {"w_gu", w_gu, true, false},
                         {"w_down", w_down, true, false}, {"offsets", offsets, true, false},
                         {"h", h, !rc, rc},               {"a", a, !rc, rc},
                         {"y", y, true, false}};
  st = validate_ptrs(args, 7, &why);
  if (st != MOE_OK) return report(st, why);
  const WorkspaceLayout w = workspace_layout(s);
  st = validate_workspace(ws, ws_bytes, w.gemm_fwd_total, &why);
  if (st != MOE_OK) return report(st, why);
  GroupedFfnArgs fa = ffn_args(s);
  fa.x_perm = x_perm;
  fa.w_gu = w_gu;
  fa.w_down = w_down;
  fa.offsets = offsets;
  fa.h = rc ? nullptr : h;  // NULL h: the gate/up epilogue writes only a
  fa.a = rc ? ws : a;
  fa.y = y;
  hipStream_t hs = as_stream(stream);
  return hip_status(s.dtype == MOE_DTYPE_BF16 ? launch_ffn_fwd_bf16(fa, hs) : launch_ffn_fwd_f32(fa, hs),
                    "grouped_gemm_fwd");
}

moe_status moe_unpermute_combine(const moe_shape *shape, const void *y, const float *topk_w,
                                 const int32_t *row_of_slot, void *out, moe_stream_t stream) {
  moe::AbiRange range("moe_unpermute_combine");
  std::string why;
  moe_status st = validate_shape(shape, &why);
  if (st != MOE_OK) return report(st, why);
  const moe_shape &s = *shape;
  if (s.T == 0) return MOE_OK;
  const PtrArg args[] = {{"y", y, true, false}, {"topk_w", topk_w, true, false},
                         {"row_of_slot", row_of_slot, true, false}, {"out", out, true, false}};
  st = validate_ptrs(args, 4, &why);
  if (st != MOE_OK) return report(st, why);
  return hip_status(
      launch_combine(y, topk_w, row_of_slot, out, s.T, s.d, s.k, s.dtype == MOE_DTYPE_BF16, as_stream(stream)),
      "unpermute_combine");
}

moe_status moe_unpermute_combine_bwd(const moe_shape *shape, const void *dout, const void *y, const float *topk_w,
                                     const int32_t *row_of_slot, void *dy, float *dtopk_w, moe_stream_t stream) {
  moe::AbiRange range("moe_unpermute_combine_bwd");
  std::string why;
  moe_status st = validate_shape(shape, &why);
  if (st != MOE_OK) return report(st, why);
  const moe_shape &s = *shape;
  if (s.T == 0) return MOE_OK;
  const PtrArg args[] = {{"dout", dout, true, false},       {"y", y, true, false},
                         {"topk_w", topk_w, true, false},   {"row_of_slot", row_of_slot, true, false},
                         {"dy", dy, true, false},           {"dtopk_w", dtopk_w, true, false}};
  st = validate_ptrs(args, 6, &why);
  if (st != MOE_OK) return report(st, why);
  return hip_status(launch_combine_bwd(dout, y, topk_w, row_of_slot, dy, dtopk_w, s.T, s.d, s.k,
                                       s.dtype == MOE_DTYPE_BF16, as_stream(stream)),
                    "unpermute_combine_bwd");
}

moe_status moe_route_bwd(const moe_shape *shape, const float *dtopk_w, const float *logits, const int32_t *topk_idx,
                         const float *topk_w, const void *x, const void *w_router, float *dlogits, float *dx_router,
                         float *dw_router, void *ws, size_t ws_bytes, moe_stream_t stream) {
  moe::AbiRange range("moe_route_bwd");
  std::string why;
  moe_status st = validate_shape(shape, &why);
  if (st != MOE_OK) return report(st, why);
  const moe_shape &s = *shape;
  if (s.T == 0) return MOE_OK;
  const bool router = w_router != nullptr;
  const PtrArg args[] = {
      {"dtopk_w", dtopk_w, true, false},  {"logits", logits, true, false},
      {"topk_idx", topk_idx, true, false}, {"topk_w", topk_w, true, false},
      {"x", x, router, !router},           {"w_router", w_router, false, false},
      {"dlogits", dlogits, true, false},   {"dx_router", dx_router, router, !router},
      {"dw_router", dw_router, router, !router},
  };
  st = validate_ptrs(args, sizeof(args) / sizeof(args[0]), &why);
  if (st != MOE_OK) return report(st, why);
  const WorkspaceLayout w = workspace_layout(s);
  if (router) {
    st = validate_workspace(ws, ws_bytes, w.route_total, &why);
    if (st != MOE_OK) return report(st, why);
  }
  hipStream_t hs = as_stream(stream);
  st = hip_status(launch_route_bwd(dtopk_w, logits, topk_idx, topk_w, dlogits, s.T, s.E, s.k,
                                   (s.flags & MOE_FLAG_RENORM) != 0, (s.flags & MOE_FLAG_ACCUMULATE_DLOGITS) != 0,
                                   hs),
                  "route_bwd");
  if (st != MOE_OK || !router) return st;
  float *partial = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + w.route_blk_cnt);
  return hip_status(launch_router_bwd(dlogits, x, w_router, dx_router, dw_router, partial, s.T, s.d, s.E,
                                      s.dtype == MOE_DTYPE_BF16, hs),
                    "router_bwd");
}

moe_status moe_grouped_gemm_bwd(const moe_shape *shape, const void *dy, const void *x_perm, const void *h,
                                const void *a, const void *w_gu, const void *w_down, const int32_t *offsets,
                                void *dx_perm, float *dw_gu, float *dw_down, void *ws, size_t ws_bytes,
                                moe_stream_t stream) {
  moe::AbiRange range("moe_grouped_gemm_bwd");
  std::string why;
  moe_status st = validate_shape(shape, &why);
  if (st != MOE_OK) return report(st, why);
  const moe_shape &s = *shape;
  if (s.T == 0) return MOE_OK;
  const bool rc = (s.flags & MOE_FLAG_RECOMPUTE) != 0;
  const PtrArg args[] = {{"dy", dy, true, false},         {"x_perm", x_perm, true, false},
                         {"h", h, !rc, rc},               {"a", a, !rc, rc},
                         {"w_gu", w_gu, true, false},     {"w_down", w_down, true, false},
                         {"offsets", offsets, true, false}, {"dx_perm", dx_perm, true, false},
                         {"dw_gu", dw_gu, true, false},   {"dw_down", dw_down, true, false}};
  st = validate_ptrs(args, 10, &why);
  if (st != MOE_OK) return report(st, why);
  const WorkspaceLayout w = workspace_layout(s);
  st = validate_workspace(ws, ws_bytes, w.gemm_bwd_total, &why);
  if (st != MOE_OK) return report(st, why);
  GroupedFfnArgs fa = ffn_args(s);
  fa.dy = dy;
  fa.x_perm = x_perm;
  fa.h = const_cast<void *>(h);
  fa.a = const_cast<void *>(a);
  fa.w_gu = w_gu;
  fa.w_down = w_down;
  fa.offsets = offsets;
  fa.dx_perm = dx_perm;
  fa.dw_gu = dw_gu;
  fa.dw_down = dw_down;
  fa.dh = ws;
  fa.order = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(ws) + w.gemm_bwd_dh);
  hipStream_t hs = as_stream(stream);
  const bool bf16 = s.dtype == MOE_DTYPE_BF16;
  if (rc) {
    // h and a again from x_perm; dH then overwrites h tile by tile (each
    // workgroup of the dgrad reads the h tile it later writes, nobody else).
    fa.h = ws;
    fa.a = reinterpret_cast<char *>(ws) + w.gemm_bwd_dh + w.gemm_bwd_order;
    st = hip_status(bf16 ? launch_ffn_recompute_bf16(fa, hs) : launch_ffn_recompute_f32(fa, hs),
                    "grouped_gemm_bwd (recompute)");
    if (st != MOE_OK) return st;
  }
  return hip_status(bf16 ? launch_ffn_bwd_bf16(fa, hs) : launch_ffn_bwd_f32(fa, hs), "grouped_gemm_bwd");
}

moe_status moe_permute_bwd(const moe_shape *shape, const void *dx_perm, const int32_t *row_of_slot,
                           const float *dx_extra, void *dx, moe_stream_t stream) {
  moe::AbiRange range("moe_permute_bwd");
  std::string why;
  moe_status st = validate_shape(shape, &why);
  if (st != MOE_OK) return report(st, why);
  const moe_shape &s = *shape;
  if (s.T == 0) return MOE_OK;
  const PtrArg args[] = {{"dx_perm", dx_perm, true, false}, {"row_of_slot", row_of_slot, true, false},
                         {"dx_extra", dx_extra, false, false}, {"dx", dx, true, false}};
  st = validate_ptrs(args, 4, &why);
  if (st != MOE_OK) return report(st, why);
  return hip_status(launch_permute_bwd(dx_perm, row_of_slot, dx_extra, dx, s.T, s.d, s.k, s.dtype == MOE_DTYPE_BF16,
                                       as_stream(stream)),
                    "permute_bwd");
}

moe_status moe_aux_loss(const moe_shape *shape, const float *logits, const int32_t *counts,
                        const moe_aux_config *cfg, float *losses, float *metrics, float *dlogits, void *ws,
                        size_t ws_bytes, moe_stream_t stream) {
  moe::AbiRange range("moe_aux_loss");
  std::string why;
  moe_status st = validate_shape(shape, &why);
  if (st != MOE_OK) return report(st, why);
  st = validate_aux(cfg, &why);
  if (st != MOE_OK) return report(st, why);
  const moe_shape &s = *shape;
  if (!losses && !metrics && (s.T == 0 || !dlogits)) return MOE_OK;
  if (s.T == 0) {
    // an empty microbatch contributes zero losses; only the outputs asked for are written
    const PtrArg outs[] = {{"losses", losses, false, false}, {"metrics", metrics, false, false}};
    st = validate_ptrs(outs, 2, &why);
    if (st != MOE_OK) return report(st, why);
    return hip_status(launch_aux_loss(nullptr, nullptr, losses, metrics, nullptr, nullptr, 0, s.E, s.k,
                                      cfg->balance_coef, cfg->z_coef, false, as_stream(stream)),
                      "aux_loss");
  }
  const PtrArg args[] = {{"logits", logits, true, false},  {"counts", counts, true, false},
                         {"losses", losses, false, false}, {"metrics", metrics, false, false},
                         {"dlogits", dlogits, false, false}};
  st = validate_ptrs(args, 5, &why);
  if (st != MOE_OK) return report(st, why);
  const WorkspaceLayout w = workspace_layout(s);
  st = validate_workspace(ws, ws_bytes, w.route_aux, &why);
  if (st != MOE_OK) return report(st, why);
  return hip_status(launch_aux_loss(logits, counts, losses, metrics, dlogits, static_cast<float *>(ws), s.T, s.E, s.k,
                                    cfg->balance_coef, cfg->z_coef, (cfg->flags & MOE_AUX_ACCUMULATE) != 0,
                                    as_stream(stream)),
                    "aux_loss");
}

moe_status moe_adamw_step(const moe_adamw_config *cfg, int64_t n, float *param, float *grad, float *exp_avg,
                          float *exp_avg_sq, void *param_bf16, moe_stream_t stream) {
  moe::AbiRange range("moe_adamw_step");
  std::string why;
  moe_status st = validate_adamw(cfg, n, &why);
  if (st != MOE_OK) return report(st, why);
  if (n == 0) return MOE_OK;
  const PtrArg args[] = {{"param", param, true, false},     {"grad", grad, true, false},
                         {"exp_avg", exp_avg, true, false}, {"exp_avg_sq", exp_avg_sq, true, false},
                         {"param_bf16", param_bf16, false, false}};
  st = validate_ptrs(args, 5, &why);
  if (st != MOE_OK) return report(st, why);
  // bias corrections in double, then rounded once to fp32
  const double bc1 = 1.0 - std::pow((double)cfg->beta1, (double)cfg->step);
  const double bc2 = 1.0 - std::pow((double)cfg->beta2, (double)cfg->step);
  if (!(bc1 > 0.0) || !(bc2 > 0.0))
    return report(MOE_ERR_INVALID_ARGUMENT, "bias correction underflows to zero (beta too close to 0 at this step?)");
  AdamwLaunch a;
  a.theta = param;
  a.grad = grad;
  a.m = exp_avg;
  a.v = exp_avg_sq;
  a.lowp = param_bf16;
  a.n = n;
  a.b1 = cfg->beta1;
  a.b2 = cfg->beta2;
  a.decay = (float)(1.0 - (double)cfg->lr * (double)cfg->weight_decay);
  a.step_size = (float)((double)cfg->lr / bc1);
  a.bc2_sqrt = (float)std::sqrt(bc2);
  a.eps = cfg->eps;
  a.scale = cfg->grad_scale;
  a.zero_grad = (cfg->flags & MOE_ADAMW_ZERO_GRAD) != 0;
  return hip_status(launch_adamw(a, as_stream(stream)), "adamw_step");
}

moe_status moe_ep_send_plan(const moe_shape *shape, int32_t ep, const int32_t *counts, const int32_t *offsets,
                            int32_t *send_counts, int32_t *send_offsets, moe_stream_t stream) {
  moe::AbiRange range("moe_ep_send_plan");
  std::string why;
  moe_status st = validate_shape(shape, &why);
  if (st != MOE_OK) return report(st, why);
  const moe_shape &s = *shape;
  if (ep < 1 || ep > kEpMaxRanks || s.E % ep != 0)
    return report(MOE_ERR_UNSUPPORTED, "moe_ep_send_plan: ep outside [1, MOE_EP_MAX_RANKS] or not dividing E");
  const bool empty = s.T == 0;
  const PtrArg args[] = {{"counts", counts, !empty, false},
                         {"offsets", offsets, !empty, false},
                         {"send_counts", send_counts, true, false},
                         {"send_offsets", send_offsets, true, false}};
  st = validate_ptrs(args, 4, &why);
  if (st != MOE_OK) return report(st, why);
  return hip_status(launch_ep_send_plan(counts, offsets, send_counts, send_offsets, ep, s.E / ep, empty,
                                        as_stream(stream)),
                    "ep_send_plan");
}

moe_status moe_ep_recv_plan(int32_t ep, int32_t e_local, int64_t rows_cap, const int32_t *recv_counts,
                            int32_t *local_counts, int32_t *local_offsets, int32_t *recv_offsets,
                            int32_t *regroup_row, moe_stream_t stream) {
  moe::AbiRange range("moe_ep_recv_plan");
  std::string why;
  moe_status st = validate_ep(ep, e_local, 0, 0, rows_cap, &why);
  if (st != MOE_OK) return report(st, why);
  const PtrArg args[] = {{"recv_counts", recv_counts, true, false},
                         {"local_counts", local_counts, true, false},
                         {"local_offsets", local_offsets, true, false},
                         {"recv_offsets", recv_offsets, true, false},
                         {"regroup_row", regroup_row, rows_cap > 0, false}};
  st = validate_ptrs(args, 5, &why);
  if (st != MOE_OK) return report(st, why);
  return hip_status(launch_ep_recv_plan(recv_counts, local_counts, local_offsets, recv_offsets, regroup_row, rows_cap,
                                        ep, e_local, as_stream(stream)),
                    "ep_recv_plan");
}

moe_status moe_ep_regroup(int32_t d, int32_t dtype, int64_t rows_cap, int32_t ep, const int32_t *recv_offsets,
                          const int32_t *regroup_row, const void *src, void *dst, int32_t reverse,
                          moe_stream_t stream) {
  moe::AbiRange range("moe_ep_regroup");
  std::string why;
  moe_status st = validate_ep(ep, 1, d, dtype, rows_cap, &why);
  if (st != MOE_OK) return report(st, why);
  if (d == 0) return report(MOE_ERR_INVALID_ARGUMENT, "moe_ep_regroup: d must be positive");
  if (rows_cap == 0) return MOE_OK;
  const PtrArg args[] = {{"recv_offsets", recv_offsets, true, false},
                         {"regroup_row", regroup_row, true, false},
                         {"src", src, true, false},
                         {"dst", dst, true, false}};
  st = validate_ptrs(args, 4, &why);
  if (st != MOE_OK) return report(st, why);
  const size_t es = dtype == MOE_DTYPE_BF16 ? 2 : 4;
  const char *a = static_cast<const char *>(src), *b = static_cast<const char *>(dst);
  const size_t bytes = (size_t)rows_cap * (size_t)d * es;
  if (a < b + bytes && b < a + bytes) return report(MOE_ERR_INVALID_ARGUMENT, "moe_ep_regroup: src and dst overlap");
  return hip_status(launch_ep_regroup(src, dst, regroup_row, recv_offsets + ep, rows_cap, d, dtype == MOE_DTYPE_BF16,
                                      reverse != 0, as_stream(stream)),
                    "ep_regroup");
}

moe_status moe_ep_exchange_counts_loopback(int32_t ep, int32_t e_local, const int32_t *const *send_counts,
                                           int32_t *const *recv_counts, moe_stream_t stream) {
  moe::AbiRange range("moe_ep_exchange_counts_loopback");
  std::string why;
  moe_status st = validate_ep(ep, e_local, 0, 0, 0, &why);
  if (st != MOE_OK) return report(st, why);
  if (!send_counts || !recv_counts) return report(MOE_ERR_INVALID_ARGUMENT, "pointer arrays are NULL");
  EpPtrs sp{}, rp{};
  for (int r = 0; r < ep; ++r) {
    const PtrArg args[] = {{"send_counts[r]", send_counts[r], true, false},
                           {"recv_counts[r]", recv_counts[r], true, false}};
    st = validate_ptrs(args, 2, &why);
    if (st != MOE_OK) return report(st, why);
    sp.p[r] = const_cast<int32_t *>(send_counts[r]);
    rp.p[r] = recv_counts[r];
  }
  return hip_status(launch_ep_exchange_counts(sp, rp, ep, e_local, as_stream(stream)), "ep_exchange_counts");
}

moe_status moe_ep_exchange_loopback(int32_t ep, int32_t d, int32_t dtype, void *const *send_bufs,
                                    const int64_t *send_caps, const int32_t *const *send_offsets,
                                    void *const *recv_bufs, const int64_t *recv_caps,
                                    const int32_t *const *recv_offsets, const int32_t *const *regroup_rows,
                                    int32_t reverse, moe_stream_t stream) {
  moe::AbiRange range("moe_ep_exchange_loopback");
  std::string why;
  moe_status st = validate_ep(ep, 1, d, dtype, 0, &why);
  if (st != MOE_OK) return report(st, why);
  if (d == 0) return report(MOE_ERR_INVALID_ARGUMENT, "moe_ep_exchange_loopback: d must be positive");
  if (!send_bufs || !send_caps || !send_offsets || !recv_bufs || !recv_caps || !recv_offsets)
    return report(MOE_ERR_INVALID_ARGUMENT, "pointer arrays are NULL");
  EpPtrs dst{}, roff{}, rgp{};
  EpCaps cap{};
  for (int r = 0; r < ep; ++r) {
    st = validate_ep(ep, 1, d, dtype, send_caps[r], &why);
    if (st == MOE_OK) st = validate_ep(ep, 1, d, dtype, recv_caps[r], &why);
    if (st != MOE_OK) return report(st, why);
    const PtrArg args[] = {{"send_bufs[r]", send_bufs[r], send_caps[r] > 0, false},
                           {"send_offsets[r]", send_offsets[r], true, false},
                           {"recv_bufs[r]", recv_bufs[r], recv_caps[r] > 0, false},
                           {"recv_offsets[r]", recv_offsets[r], true, false}};
    st = validate_ptrs(args, 4, &why);
    if (st != MOE_OK) return report(st, why);
    dst.p[r] = recv_bufs[r];
    roff.p[r] = const_cast<int32_t *>(recv_offsets[r]);
    cap.n[r] = recv_caps[r];
    if (regroup_rows) {
      const PtrArg rg[] = {{"regroup_rows[r]", regroup_rows[r], recv_caps[r] > 0, false}};
      st = validate_ptrs(rg, 1, &why);
      if (st != MOE_OK) return report(st, why);
      rgp.p[r] = const_cast<int32_t *>(regroup_rows[r]);
    }
  }
  hipStream_t hs = as_stream(stream);
  for (int s = 0; s < ep; ++s) {
    st = hip_status(launch_ep_exchange_rows(send_bufs[s], send_offsets[s], send_caps[s], dst, roff, rgp, cap, s, ep,
                                            d, dtype == MOE_DTYPE_BF16, reverse != 0, hs),
                    "ep_exchange_rows");
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

static int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

int64_t moe_peak_mfma_size(void) {
  const int cus = device_cus();
  return cus > 0 ? (int64_t)peak_mfma_threads(cus) : 0;
}

moe_status moe_peak_mfma(float *out, int32_t iters, double *flops, moe_stream_t stream) {
  if (!out || !flops) return report(MOE_ERR_INVALID_ARGUMENT, "moe_peak_mfma: out and flops are required");
  if (iters < 1) return report(MOE_ERR_INVALID_ARGUMENT, "moe_peak_mfma: iters < 1");
  if (((uintptr_t)out & 15u) != 0) return report(MOE_ERR_MISALIGNED, "moe_peak_mfma: out is not 16-byte aligned");
  const int cus = device_cus();
  if (cus <= 0) return report(MOE_ERR_HIP, "moe_peak_mfma: no device");
  *flops = peak_mfma_flops(cus, iters);
  return hip_status(launch_peak_mfma(out, cus, iters, as_stream(stream)), "peak_mfma");
}

moe_status moe_peak_copy(const void *src, void *dst, int64_t bytes, moe_stream_t stream) {
  if (!src || !dst) return report(MOE_ERR_INVALID_ARGUMENT, "moe_peak_copy: src and dst are required");
  if (bytes <= 0 || bytes % 16 != 0)
    return report(MOE_ERR_INVALID_ARGUMENT, "moe_peak_copy: bytes must be a positive multiple of 16");
  if ((((uintptr_t)src | (uintptr_t)dst) & 15u) != 0)
    return report(MOE_ERR_MISALIGNED, "moe_peak_copy: src or dst is not 16-byte aligned");
  const char *s0 = static_cast<const char *>(src), *d0 = static_cast<const char *>(dst);
  if (s0 < d0 + bytes && d0 < s0 + bytes) return report(MOE_ERR_INVALID_ARGUMENT, "moe_peak_copy: buffers overlap");
  if (bytes / 16 > (int64_t)0xffffffff * 256) return report(MOE_ERR_UNSUPPORTED, "moe_peak_copy: too many bytes");
  return hip_status(launch_peak_copy(src, dst, bytes, as_stream(stream)), "peak_copy");
}

moe_status moe_profiler_enable(int on) {
  g_prof.on.store(on != 0);
  return MOE_OK;
}

moe_status moe_profiler_reset(void) {
  std::lock_guard<std::mutex> lock(g_prof.mu);
  for (size_t i = 0; i < g_prof.entries.size(); ++i) g_prof.drain((int)i);
  g_prof.entries.clear();
  return MOE_OK;
}

int moe_profiler_count(void) {
  std::lock_guard<std::mutex> lock(g_prof.mu);
  return (int)g_prof.entries.size();
}

moe_status moe_profiler_read(int i, const char **name, int64_t *launches, double *total_ms) {
  std::lock_guard<std::mutex> lock(g_prof.mu);
  if (i < 0 || i >= (int)g_prof.entries.size()) return report(MOE_ERR_INVALID_ARGUMENT, "profiler index out of range");
  g_prof.drain(i);
  const ProfEntry &en = g_prof.entries[i];
  if (name) *name = en.name;
  if (launches) *launches = en.launches;
  if (total_ms) *total_ms = en.ms;
  return MOE_OK;
}

}  // extern "C"
