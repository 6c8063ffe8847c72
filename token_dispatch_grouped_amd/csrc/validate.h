// Host-side argument validation and workspace sizing for the C ABI. Pure
// C++ (no HIP), so it can be built and unit-tested without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "moe.h"

namespace moe {

// Tile sizes the launchers use; validation checks that grids fit.
constexpr int kRouteTokens = 64;        // tokens per top-k workgroup (one wavefront)
constexpr int kRouterChunksMax = 32;    // router weight-gradient partial sums
constexpr int kGemmBM = 256;            // bf16 grouped GEMM rows per tile
constexpr int kGemmBN = 256;            // bf16 grouped GEMM columns per tile
constexpr int kGemmGroupM = 4;          // row tiles per group in the ragged-M tile order
constexpr int kGemmF32Tile = 16;        // fp32 grouped GEMM tile edge
constexpr int kAuxMaxBlocks = 1024;     // partial rows of the auxiliary-loss pass
// Static per-GPU scratch of moe_route_noalloc: the per-workgroup expert
// histograms of the route pass, ceil(T / kRouteTokens) * E int32.
constexpr size_t kRouteScratchBytes = (size_t)16 << 20;
constexpr int kEpMaxRanks = 8;          // expert-parallel ranks of the exchange stand-in (one node)

struct WorkspaceLayout {
  size_t route_blk_cnt;   // bytes of the per-workgroup expert histograms
  size_t route_partial;   // bytes of router weight-gradient partial sums
  size_t route_aux;       // bytes of the auxiliary-loss partial rows (shares the route workspace)
  size_t route_total;
  size_t gemm_fwd_total;  // recompute: a [R,F] at offset 0; else nothing
  size_t gemm_bwd_dh;     // bytes of dH (recompute: the recomputed h first)
  size_t gemm_bwd_order;  // bytes of the expert order (int32 [E])
  size_t gemm_bwd_a;      // recompute: bytes of the recomputed a; else 0
  size_t gemm_bwd_total;  // dh | order | a
};

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tokens per workgroup of the auxiliary-loss pass: at least kAuxMinTokens
// (512 workgroups at 32k tokens), at most kAuxMaxBlocks workgroups.
constexpr int kAuxMinTokens = 64;
inline int aux_tokens_per_block(int64_t T) {
  int64_t tpb = ceil_div(T, kAuxMaxBlocks);
  if (tpb < kAuxMinTokens) tpb = kAuxMinTokens;
  return (int)tpb;
}

// Validates the shape alone. On failure writes a message to *why.
moe_status validate_shape(const moe_shape *s, std::string *why);

// Workspace layout of a (validated) shape.
WorkspaceLayout workspace_layout(const moe_shape &s);

// One pointer argument: `needed` tells whether the call reads or writes it.
// NULL where needed -> MOE_ERR_INVALID_ARGUMENT; non-NULL where it must be
// NULL (must_be_null) -> MOE_ERR_INVALID_ARGUMENT; not 16-byte aligned ->
// MOE_ERR_MISALIGNED.
struct PtrArg {
  const char *name;
  const void *ptr;
  bool needed;
  bool must_be_null;
};
moe_status validate_ptrs(const PtrArg *args, int n, std::string *why);

// AdamW scalars and element count (see moe_adamw_step).
moe_status validate_adamw(const moe_adamw_config *cfg, int64_t n, std::string *why);

// Auxiliary-loss coefficients and flags (see moe_aux_loss).
moe_status validate_aux(const moe_aux_config *cfg, std::string *why);

// Expert-parallel exchange sizes: 1 <= ep <= kEpMaxRanks, e_local >= 1,
// ep*e_local <= 256; d a positive multiple of 64 (<= 65536) and dtype valid
// when d > 0 is given; capacities >= 0 and below 2^31 rows.
moe_status validate_ep(int32_t ep, int32_t e_local, int32_t d, int32_t dtype, int64_t rows_cap, std::string *why);

// Workspace check: NULL or short -> MOE_ERR_WORKSPACE (a zero requirement
// accepts anything).
moe_status validate_workspace(const void *ws, size_t have, size_t need, std::string *why);

}  // namespace moe
