// Host-side validation of every C-ABI argument, done before anything is
// launched. Unsupported configurations are rejected explicitly and up front
// (Support combined expert and data parallelism in TrainerRank, Current
// behavior and Desired behavior), and every argument is checked before any
// is consumed (review note on Add MoE expert parallel training runtime).
#include "validate.h"

#include <cmath>

#include <stdio.h>

namespace moe {

static moe_status fail(std::string *why, moe_status st, const char *msg) {
  if (why) *why = msg;
  return st;
}

moe_status validate_shape(const moe_shape *s, std::string *why) {
  if (!s) return fail(why, MOE_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (s->T < 0) return fail(why, MOE_ERR_INVALID_ARGUMENT, "T < 0");
  if (s->d <= 0 || s->E <= 0 || s->k <= 0 || s->F <= 0)
    return fail(why, MOE_ERR_INVALID_ARGUMENT, "d, E, k and F must be positive");
  if (s->k > s->E) return fail(why, MOE_ERR_INVALID_ARGUMENT, "k > E");
  if (s->dtype != MOE_DTYPE_F32 && s->dtype != MOE_DTYPE_BF16)
    return fail(why, MOE_ERR_UNSUPPORTED, "dtype must be MOE_DTYPE_F32 or MOE_DTYPE_BF16");
  if (s->flags & ~(uint32_t)(MOE_FLAG_RENORM | MOE_FLAG_RECOMPUTE | MOE_FLAG_ACCUMULATE_DLOGITS))
    return fail(why, MOE_ERR_UNSUPPORTED, "unknown flag bits");
  if (s->E > 256) return fail(why, MOE_ERR_UNSUPPORTED, "E > 256");
  if (s->k > 16) return fail(why, MOE_ERR_UNSUPPORTED, "k > 16");
  if (s->d % 64 != 0 || s->F % 64 != 0) return fail(why, MOE_ERR_UNSUPPORTED, "d and F must be multiples of 64");
  if (s->d > 65536 || s->F > 65536) return fail(why, MOE_ERR_UNSUPPORTED, "d or F > 65536");
  const int64_t R = s->T * (int64_t)s->k;
  if (s->T > ((int64_t)1 << 31) || R >= ((int64_t)1 << 31)) return fail(why, MOE_ERR_UNSUPPORTED, "T*k >= 2^31");
  // every tile count must fit in 2^31 - 1; the bf16 bounds round like the
  // launchers: ragged-M row slots up to whole row-tile groups and the logical
  // tile count up to a multiple of 8, weight-gradient grids up to a multiple
  // of 64
  const int64_t lim = ((int64_t)1 << 31) - 1;
  const int64_t wide = s->d > 2 * (int64_t)s->F ? s->d : 2 * (int64_t)s->F;
  int64_t gemm_blocks;
  int64_t gemm_threads;  // threads of the largest grouped-GEMM launch that is not persistent
  if (s->dtype == MOE_DTYPE_BF16) {
    const int64_t slots = ceil_div(R / kGemmBM + s->E, kGemmGroupM) * kGemmGroupM;
    gemm_blocks = ceil_div(slots * ceil_div(wide, kGemmBN / 2), 8) * 8;
    const int64_t wg = ceil_div((int64_t)s->E * ceil_div(wide, kGemmBM) * ceil_div(wide, kGemmBN), 64) * 64;
    if (wg > gemm_blocks) gemm_blocks = wg;
    gemm_threads = wg * 512;  // the ragged-M products run one 512-thread workgroup per CU
  } else {
    gemm_blocks = (R / kGemmF32Tile + s->E) * ceil_div(wide, kGemmF32Tile);
    const int64_t wg = (int64_t)s->E * ceil_div(wide, kGemmF32Tile) * ceil_div(wide, kGemmF32Tile);
    if (wg > gemm_blocks) gemm_blocks = wg;
    gemm_threads = gemm_blocks * 256;
  }
  const int64_t vec = s->dtype == MOE_DTYPE_BF16 ? 8 : 4;
  const int64_t mem_blocks = ceil_div(s->T * (s->d / vec), 256);
  if (gemm_blocks > lim || mem_blocks > lim) return fail(why, MOE_ERR_UNSUPPORTED, "problem too large for one launch");
  // a grid dimension holds fewer than 2^32 threads: the per-token launches
  // (256 threads per token at most), the one-thread-per-chunk memory kernels
  // and the non-persistent grouped GEMM grids
  const int64_t items = (int64_t)1 << 32;
  if (s->T * 256 >= items || s->T * (s->d / vec) >= items || gemm_threads >= items)
    return fail(why, MOE_ERR_UNSUPPORTED, "problem too large for one launch (2^32 threads per grid dimension)");
  return MOE_OK;
}

WorkspaceLayout workspace_layout(const moe_shape &s) {
  WorkspaceLayout w{};
  const int64_t nblk = ceil_div(s.T, kRouteTokens);
  w.route_blk_cnt = align256((size_t)nblk * (size_t)s.E * 4);
  int64_t chunk_tokens = ceil_div(s.T, kRouterChunksMax);
  if (chunk_tokens < 256) chunk_tokens = 256;
  const int64_t nchunk = ceil_div(s.T, chunk_tokens);
  w.route_partial = align256((size_t)nchunk * (size_t)s.E * (size_t)s.d * 4);
  const int64_t aux_blocks = ceil_div(s.T, aux_tokens_per_block(s.T));
  w.route_aux = align256((size_t)aux_blocks * ((size_t)s.E + 3) * 4);
  w.route_total = w.route_blk_cnt + w.route_partial;
  if (w.route_aux > w.route_total) w.route_total = w.route_aux;
  const size_t es = s.dtype == MOE_DTYPE_BF16 ? 2 : 4;
  const size_t R = (size_t)s.T * (size_t)s.k;
  const bool recompute = (s.flags & MOE_FLAG_RECOMPUTE) != 0;
  w.gemm_fwd_total = recompute ? align256(R * (size_t)s.F * es) : 0;
  w.gemm_bwd_dh = align256(R * 2 * (size_t)s.F * es);
  w.gemm_bwd_order = align256((size_t)s.E * 4);
  w.gemm_bwd_a = recompute ? align256(R * (size_t)s.F * es) : 0;
  w.gemm_bwd_total = w.gemm_bwd_dh + w.gemm_bwd_order + w.gemm_bwd_a;
  return w;
}

moe_status validate_ptrs(const PtrArg *args, int n, std::string *why) {
  for (int i = 0; i < n; ++i) {
    const PtrArg &a = args[i];
    char buf[160];
    if (a.needed && !a.ptr) {
      snprintf(buf, sizeof buf, "%s is NULL", a.name);
      return fail(why, MOE_ERR_INVALID_ARGUMENT, buf);
    }
    if (a.must_be_null && a.ptr) {
      snprintf(buf, sizeof buf, "%s must be NULL in this mode", a.name);
      return fail(why, MOE_ERR_INVALID_ARGUMENT, buf);
    }
  }
  for (int i = 0; i < n; ++i) {
    const PtrArg &a = args[i];
    if (a.ptr && ((uintptr_t)a.ptr & 15u) != 0) {
      char buf[160];
      snprintf(buf, sizeof buf, "%s is not 16-byte aligned", a.name);
      return fail(why, MOE_ERR_MISALIGNED, buf);
    }
  }
  return MOE_OK;
}

moe_status validate_workspace(const void *ws, size_t have, size_t need, std::string *why) {
  if (need == 0) return MOE_OK;
  if (!ws) return fail(why, MOE_ERR_WORKSPACE, "workspace is NULL");
  if (((uintptr_t)ws & 15u) != 0) return fail(why, MOE_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  if (have < need) {
    char buf[160];
    snprintf(buf, sizeof buf, "workspace too small: %zu bytes given, %zu needed", have, need);
    return fail(why, MOE_ERR_WORKSPACE, buf);
  }
  return MOE_OK;
}

moe_status validate_adamw(const moe_adamw_config *c, int64_t n, std::string *why) {
  if (!c) return fail(why, MOE_ERR_INVALID_ARGUMENT, "adamw config is NULL");
  if (n < 0) return fail(why, MOE_ERR_INVALID_ARGUMENT, "negative element count");
  // eight elements per thread: 2^35 elements fill a grid of 2^32 threads
  if (n >= ((int64_t)1 << 35)) return fail(why, MOE_ERR_UNSUPPORTED, "element count >= 2^35");
  if (c->flags & ~(uint32_t)MOE_ADAMW_ZERO_GRAD) return fail(why, MOE_ERR_UNSUPPORTED, "unknown adamw flag bits");
  const float vals[] = {c->lr, c->beta1, c->beta2, c->eps, c->weight_decay, c->grad_scale};
  for (float v : vals)
    if (!std::isfinite(v)) return fail(why, MOE_ERR_INVALID_ARGUMENT, "non-finite adamw scalar");
  if (c->lr < 0.f) return fail(why, MOE_ERR_INVALID_ARGUMENT, "lr < 0");
  if (c->beta1 < 0.f || c->beta1 >= 1.f || c->beta2 < 0.f || c->beta2 >= 1.f)
    return fail(why, MOE_ERR_INVALID_ARGUMENT, "beta outside [0, 1)");
  if (c->eps <= 0.f) return fail(why, MOE_ERR_INVALID_ARGUMENT, "eps <= 0");
  if (c->weight_decay < 0.f) return fail(why, MOE_ERR_INVALID_ARGUMENT, "weight_decay < 0");
  if (c->step < 1) return fail(why, MOE_ERR_INVALID_ARGUMENT, "step < 1");
  return MOE_OK;
}

moe_status validate_ep(int32_t ep, int32_t e_local, int32_t d, int32_t dtype, int64_t rows_cap, std::string *why) {
  if (ep < 1 || ep > kEpMaxRanks) return fail(why, MOE_ERR_UNSUPPORTED, "ep outside [1, MOE_EP_MAX_RANKS]");
  if (e_local < 1) return fail(why, MOE_ERR_INVALID_ARGUMENT, "e_local < 1");
  if ((int64_t)ep * e_local > 256) return fail(why, MOE_ERR_UNSUPPORTED, "ep * e_local > 256");
  if (d != 0) {
    if (d < 0) return fail(why, MOE_ERR_INVALID_ARGUMENT, "d < 0");
    if (d % 64 != 0 || d > 65536) return fail(why, MOE_ERR_UNSUPPORTED, "d must be a multiple of 64, at most 65536");
    if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16)
      return fail(why, MOE_ERR_UNSUPPORTED, "dtype must be MOE_DTYPE_F32 or MOE_DTYPE_BF16");
  }
  if (rows_cap < 0) return fail(why, MOE_ERR_INVALID_ARGUMENT, "negative row capacity");
  // one 256-thread workgroup per row: 2^24 rows fill a grid of 2^32 threads
  if (rows_cap >= ((int64_t)1 << 24)) return fail(why, MOE_ERR_UNSUPPORTED, "row capacity >= 2^24");
  return MOE_OK;
}

moe_status validate_aux(const moe_aux_config *c, std::string *why) {
  if (!c) return fail(why, MOE_ERR_INVALID_ARGUMENT, "aux config is NULL");
  if (c->flags & ~(uint32_t)MOE_AUX_ACCUMULATE) return fail(why, MOE_ERR_UNSUPPORTED, "unknown aux flag bits");
  if (!std::isfinite(c->balance_coef) || !std::isfinite(c->z_coef))
    return fail(why, MOE_ERR_INVALID_ARGUMENT, "non-finite aux coefficient");
  return MOE_OK;
}

}  // namespace moe
