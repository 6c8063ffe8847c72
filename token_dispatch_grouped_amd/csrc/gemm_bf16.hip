// Host launchers of the grouped expert GEMMs in bf16 ("grouped expert
// compute", Add MoE expert parallel training runtime, Major changes): the six
// products of the SwiGLU expert FFN, forward and backward, each one launch of
// the kernel template in gemm_bf16_kernel.h, which also describes the tiling,
// the scheduling and the epilogues.
#include "gemm_bf16_kernel.h"

namespace moe {

// Experts sorted by descending row count (ties by id), so that the longest
// weight-gradient reductions start first. One workgroup, E <= 256.
__global__ __launch_bounds__(256) void expert_order_kernel(const int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ order, int E) {
  __shared__ int cnt[256];
  const int e = threadIdx.x;
  if (e < E) cnt[e] = offsets[e + 1] - offsets[e];
  __syncthreads();
  if (e >= E) return;
  const int c = cnt[e];
  int rank = 0;
  for (int o = 0; o < E; ++o) {
    const int co = cnt[o];
    rank += (co > c) || (co == c && o < e);
  }
  order[rank] = e;
}

static GemmParams base_params(const GroupedFfnArgs &a) {
  GemmParams p{};
  p.offsets = a.offsets;
  p.E = a.E;
  p.F = a.F;
  return p;
}

// Ragged-M logical tile count: an upper bound of the number of BM-row tiles
// over all experts (sum of ceil(M_e/BM) <= R/BM + E, rounded up to whole
// row-tile groups), times the column tiles. The persistent launch splits the
// real tiles it finds on the device, never more than this.
static int ragged_m_total(int64_t R, int E, int BM, int n_tiles) {
  const int64_t slots = (R / BM + E + kGroupM - 1) / kGroupM * kGroupM;
  return (int)(slots * (int64_t)n_tiles);
}

// A5: h = X_e W_gu[e]^T and a = silu(h_gate) h_up (h not stored when a.h is NULL).
static hipError_t gateup_swiglu_bf16(const GroupedFfnArgs &a, const char *name, hipStream_t s) {
  constexpr int BM = kGemmBM, BN = kGemmBN;
  LaunchScope scope(name, s);
  GemmParams p = base_params(a);
  p.A = (const bf16_t *)a.x_perm;
  p.B = (const bf16_t *)a.w_gu;
  p.C = a.h;
  p.C2 = (bf16_t *)a.a;
  p.N = a.F;
  p.K = a.d;
  p.lda = a.d;
  p.ldb = a.d;
  p.ldc = 2 * (int64_t)a.F;
  p.strideB = 2 * (int64_t)a.F * a.d;
  p.n_tiles = (a.F + BN / 2 - 1) / (BN / 2);
  p.total = ragged_m_total(a.R, a.E, BM, p.n_tiles);
  return run_dma<BM, BN, BM / 2, BN / 4, false, false, EPI_SWIGLU_FWD, false>(p, s);
}

hipError_t launch_ffn_recompute_bf16(const GroupedFfnArgs &a, hipStream_t s) {
  return gateup_swiglu_bf16(a, "gg_gateup_recompute", s);
}

hipError_t launch_ffn_fwd_bf16(const GroupedFfnArgs &a, hipStream_t s) {
  hipError_t err = gateup_swiglu_bf16(a, "gg_gateup_fwd", s);
  if (err != hipSuccess) return err;
  {
    constexpr int BM = kGemmBM, BN = kGemmBN;
    LaunchScope scope("gg_down_fwd", s);
    GemmParams p = base_params(a);
    p.A = (const bf16_t *)a.a;
    p.B = (const bf16_t *)a.w_down;
    p.C = a.y;
    p.N = a.d;
    p.K = a.F;
    p.lda = a.F;
    p.ldb = a.F;
    p.ldc = a.d;
    p.strideB = (int64_t)a.d * a.F;
    p.n_tiles = (a.d + BN - 1) / BN;
    p.total = ragged_m_total(a.R, a.E, BM, p.n_tiles);
    err = run_dma<BM, BN, BM / 2, BN / 4, false, false, EPI_STORE, false>(p, s);
  }
  return err;
}

hipError_t launch_ffn_bwd_bf16(const GroupedFfnArgs &a, hipStream_t s) {
  hipError_t err;
  {  // B3: dA = dY W_down[e], SwiGLU backward in the epilogue -> dH
    constexpr int BM = kGemmBM, BN = kGemmBN;
    LaunchScope scope("gg_down_dgrad", s);
    GemmParams p = base_params(a);
    p.A = (const bf16_t *)a.dy;
    p.B = (const bf16_t *)a.w_down;
    p.C = a.dh;
    p.H = (const bf16_t *)a.h;
    p.N = a.F;
    p.K = a.d;
    p.lda = a.d;
    p.ldb = a.F;
    p.ldc = 2 * (int64_t)a.F;
    p.strideB = (int64_t)a.d * a.F;
    p.n_tiles = (a.F + BN - 1) / BN;
    p.total = ragged_m_total(a.R, a.E, BM, p.n_tiles);
    err = run_dma<BM, BN, BM / 2, BN / 4, false, true, EPI_SWIGLU_BWD, false>(p, s);
  }
  if (err != hipSuccess) return err;
  {
    LaunchScope scope("expert_order", s);
    expert_order_kernel<<<1, 256, 0, s>>>(a.offsets, a.order, a.E);
    err = hipGetLastError();
  }
  if (err != hipSuccess) return err;
  {  // B4: dW_down[e] += dY_e^T a_e
    constexpr int BM = kGemmBM, BN = kGemmBN;
    LaunchScope scope("gg_down_wgrad", s);
    GemmParams p = base_params(a);
    p.A = (const bf16_t *)a.dy;
    p.B = (const bf16_t *)a.a;
    p.C = a.dw_down;
    p.order = a.order;
    p.M = a.d;
    p.N = a.F;
    p.lda = a.d;
    p.ldb = a.F;
    p.ldc = a.F;
    p.strideC = (int64_t)a.d * a.F;
    p.m_tiles = (a.d + BM - 1) / BM;
    p.n_tiles = (a.F + BN - 1) / BN;
    if (a.F % BN == kEdgeBN && a.d % kEdgeBM == 0) {  // F = 1408: the last 128 columns as edge tiles
      p.n_tiles = a.F / BN;
      p.mix_cols = p.n_tiles * BN;
      p.mix_mtiles = a.d / kEdgeBM;
    }
    p.total = a.E * (p.m_tiles * p.n_tiles + p.mix_mtiles);
    err = run_dma<BM, BN, BM / 2, BN / 4, true, true, EPI_ACC_F32, true>(p, s);
  }
  if (err != hipSuccess) return err;
  {  // B5: dX_perm = dH W_gu[e]
    constexpr int BM = kGemmBM, BN = kGemmBN;
    LaunchScope scope("gg_gateup_dgrad", s);
    GemmParams p = base_params(a);
    p.A = (const bf16_t *)a.dh;
    p.B = (const bf16_t *)a.w_gu;
    p.C = a.dx_perm;
    p.N = a.d;
    p.K = 2 * a.F;
    p.lda = 2 * (int64_t)a.F;
    p.ldb = a.d;
    p.ldc = a.d;
    p.strideB = 2 * (int64_t)a.F * a.d;
    p.n_tiles = (a.d + BN - 1) / BN;
    p.total = ragged_m_total(a.R, a.E, BM, p.n_tiles);
    err = run_dma<BM, BN, BM / 2, BN / 4, false, true, EPI_STORE, false>(p, s);
  }
  if (err != hipSuccess) return err;
  {  // B6: dW_gu[e] += dH^T X_e
    constexpr int BM = kGemmBM, BN = kGemmBN;
    LaunchScope scope("gg_gateup_wgrad", s);
    GemmParams p = base_params(a);
    p.A = (const bf16_t *)a.dh;
    p.B = (const bf16_t *)a.x_perm;
    p.C = a.dw_gu;
    p.order = a.order;
    p.M = 2 * a.F;
    p.N = a.d;
    p.lda = 2 * (int64_t)a.F;
    p.ldb = a.d;
    p.ldc = a.d;
    p.strideC = 2 * (int64_t)a.F * a.d;
    p.m_tiles = (2 * a.F + BM - 1) / BM;
    p.n_tiles = (a.d + BN - 1) / BN;
    p.total = a.E * p.m_tiles * p.n_tiles;
    err = run_dma<BM, BN, BM / 2, BN / 4, true, true, EPI_ACC_F32, true>(p, s);
  }
  return err;
}

}  // namespace moe
