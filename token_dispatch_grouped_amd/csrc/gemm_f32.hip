// Grouped expert GEMMs for an fp32 layer ("grouped expert compute", Add MoE
// expert parallel training runtime, Major changes).
//
// Same six products and the same device-side tiling from `offsets` as the
// bf16 path, computed with fp32 FMAs on 16x16 LDS tiles (one output per
// thread; the gate/up product keeps a gate and an up accumulator per thread
// so that the SwiGLU runs in registers). This path serves fp32 layers, where
// exactness to ~1e-6 matters more than speed.
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

enum { F32_STORE = 0, F32_SWIGLU_FWD = 1, F32_SWIGLU_BWD = 2, F32_ACC = 3 };

struct GemmParamsF {
  const float *A;
  const float *B;
  float *C;
  float *C2;         // F32_SWIGLU_FWD: the activation a
  const float *H;    // F32_SWIGLU_BWD: saved h
  const int32_t *offsets;
  int E, M, N, K;
  int64_t lda, ldb, ldc, strideB, strideC;
  int F;
  int n_tiles, m_tiles, total;
};

constexpr int kT = kGemmF32Tile;

template <bool AT, bool BT, int EPI, bool RAGGED_K>
__global__ __launch_bounds__(256) void gg_f32_kernel(GemmParamsF p) {
  __shared__ float As[kT][kT + 1];
  __shared__ float Bs[kT][kT + 1];
  __shared__ float Us[kT][kT + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int bid = blockIdx.x;
  if (bid >= p.total) return;

  int e, m0, n_tile, m_valid, kdim;
  int64_t crow0;
  const float *Ab;
  const float *Bb;
  if (!RAGGED_K) {
    n_tile = bid % p.n_tiles;
    int mt;
    if (!find_m_tile<kT>(p.offsets, p.E, bid / p.n_tiles, e, mt)) return;
    const int row0 = p.offsets[e];
    m0 = mt * kT;
    m_valid = min(kT, p.offsets[e + 1] - row0 - m0);
    crow0 = (int64_t)row0 + m0;
    Ab = p.A + crow0 * p.lda;
    Bb = p.B + (int64_t)e * p.strideB;
    kdim = p.K;
  } else {
    const int per_e = p.m_tiles * p.n_tiles;
    e = bid / per_e;
    const int r = bid - e * per_e;
    const int mt = r / p.n_tiles;
    n_tile = r - mt * p.n_tiles;
    const int row0 = p.offsets[e];
    kdim = p.offsets[e + 1] - row0;
    if (kdim <= 0) return;
    m0 = mt * kT;
    m_valid = min(kT, p.M - m0);
    crow0 = 0;
    Ab = p.A + (int64_t)row0 * p.lda;
    Bb = p.B + (int64_t)row0 * p.ldb;
  }
  const int n0 = n_tile * kT;

  float acc = 0.f, acc_up = 0.f;
  for (int k0 = 0; k0 < kdim; k0 += kT) {
    {  // A(m0 + ty, k0 + tx)
      const int m = ty, kk = k0 + tx;
      float v = 0.f;
      if (m < m_valid && kk < kdim) v = AT ? Ab[(int64_t)kk * p.lda + m0 + m] : Ab[(int64_t)m * p.lda + kk];
      As[ty][tx] = v;
    }
    {  // B(n0 + ty, k0 + tx) (and the matching up row)
      const int n = n0 + ty, kk = k0 + tx;
      float v = 0.f, u = 0.f;
      if (n < p.N && kk < kdim) {
        v = BT ? Bb[(int64_t)kk * p.ldb + n] : Bb[(int64_t)n * p.ldb + kk];
        if (EPI == F32_SWIGLU_FWD) u = Bb[(int64_t)(p.F + n) * p.ldb + kk];
      }
      Bs[ty][tx] = v;
      Us[ty][tx] = u;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kT; ++kk) {
      acc = fmaf(As[ty][kk], Bs[tx][kk], acc);
      if (EPI == F32_SWIGLU_FWD) acc_up = fmaf(As[ty][kk], Us[tx][kk], acc_up);
    }
    __syncthreads();
  }

  const int r = ty, n = n0 + tx;
  if (r >= m_valid || n >= p.N) return;
  if (EPI == F32_SWIGLU_FWD) {
    const int64_t row = crow0 + r;
    if (p.C) {  // NULL when h is not kept
      p.C[row * p.ldc + n] = acc;
      p.C[row * p.ldc + p.F + n] = acc_up;
    }
    p.C2[row * p.F + n] = silu_f(acc) * acc_up;
  } else if (EPI == F32_SWIGLU_BWD) {  // p.C may equal p.H: each element is read, then written, by one thread
    const int64_t row = crow0 + r;
    const float hg = p.H[row * p.ldc + n];
    const float hu = p.H[row * p.ldc + p.F + n];
    const float sg = 1.f / (1.f + expf(-hg));
    p.C[row * p.ldc + n] = acc * hu * sg * (1.f + hg * (1.f - sg));
    p.C[row * p.ldc + p.F + n] = acc * hg * sg;
  } else if (EPI == F32_STORE) {
    p.C[(crow0 + r) * p.ldc + n] = acc;
  } else {
    float *dst = p.C + (int64_t)e * p.strideC + (int64_t)(m0 + r) * p.ldc + n;
    *dst = *dst + acc;
  }
}

template <bool AT, bool BT, int EPI, bool RAGGED_K>
static hipError_t run_f32(const GemmParamsF &p, hipStream_t s) {
  if (p.total <= 0) return hipSuccess;
  gg_f32_kernel<AT, BT, EPI, RAGGED_K><<<dim3((unsigned)p.total), 256, 0, s>>>(p);
  return hipGetLastError();
}

static GemmParamsF base_f(const GroupedFfnArgs &a) {
  GemmParamsF p{};
  p.offsets = a.offsets;
  p.E = a.E;
  p.F = a.F;
  return p;
}

static int ragged_total_f(int64_t R, int E, int n_tiles) { return (int)((R / kT + E) * (int64_t)n_tiles); }

// h = X_e W_gu[e]^T and a = silu(h_gate) h_up (h not stored when a.h is NULL).
static hipError_t gateup_swiglu_f32(const GroupedFfnArgs &a, const char *name, hipStream_t s) {
  LaunchScope scope(name, s);
  GemmParamsF p = base_f(a);
  p.A = (const float *)a.x_perm;
  p.B = (const float *)a.w_gu;
  p.C = (float *)a.h;
  p.C2 = (float *)a.a;
  p.N = a.F;
  p.K = a.d;
  p.lda = a.d;
  p.ldb = a.d;
  p.ldc = 2 * (int64_t)a.F;
  p.strideB = 2 * (int64_t)a.F * a.d;
  p.n_tiles = (a.F + kT - 1) / kT;
  p.total = ragged_total_f(a.R, a.E, p.n_tiles);
  return run_f32<false, false, F32_SWIGLU_FWD, false>(p, s);
}

hipError_t launch_ffn_recompute_f32(const GroupedFfnArgs &a, hipStream_t s) {
  return gateup_swiglu_f32(a, "gg_gateup_recompute_f32", s);
}

hipError_t launch_ffn_fwd_f32(const GroupedFfnArgs &a, hipStream_t s) {
  hipError_t err = gateup_swiglu_f32(a, "gg_gateup_fwd_f32", s);
  if (err != hipSuccess) return err;
  {
    LaunchScope scope("gg_down_fwd_f32", s);
    GemmParamsF p = base_f(a);
    p.A = (const float *)a.a;
    p.B = (const float *)a.w_down;
    p.C = (float *)a.y;
    p.N = a.d;
    p.K = a.F;
    p.lda = a.F;
    p.ldb = a.F;
    p.ldc = a.d;
    p.strideB = (int64_t)a.d * a.F;
    p.n_tiles = (a.d + kT - 1) / kT;
    p.total = ragged_total_f(a.R, a.E, p.n_tiles);
    err = run_f32<false, false, F32_STORE, false>(p, s);
  }
  return err;
}

hipError_t launch_ffn_bwd_f32(const GroupedFfnArgs &a, hipStream_t s) {
  hipError_t err;
  {
    LaunchScope scope("gg_down_dgrad_f32", s);
    GemmParamsF p = base_f(a);
    p.A = (const float *)a.dy;
    p.B = (const float *)a.w_down;
    p.C = (float *)a.dh;
    p.H = (const float *)a.h;
    p.N = a.F;
    p.K = a.d;
    p.lda = a.d;
    p.ldb = a.F;
    p.ldc = 2 * (int64_t)a.F;
    p.strideB = (int64_t)a.d * a.F;
    p.n_tiles = (a.F + kT - 1) / kT;
    p.total = ragged_total_f(a.R, a.E, p.n_tiles);
    err = run_f32<false, true, F32_SWIGLU_BWD, false>(p, s);
  }
  if (err != hipSuccess) return err;
  {
    LaunchScope scope("gg_down_wgrad_f32", s);
    GemmParamsF p = base_f(a);
    p.A = (const float *)a.dy;
    p.B = (const float *)a.a;
    p.C = a.dw_down;
    p.M = a.d;
    p.N = a.F;
    p.lda = a.d;
    p.ldb = a.F;
    p.ldc = a.F;
    p.strideC = (int64_t)a.d * a.F;
    p.m_tiles = (a.d + kT - 1) / kT;
    p.n_tiles = (a.F + kT - 1) / kT;
    p.total = a.E * p.m_tiles * p.n_tiles;
    err = run_f32<true, true, F32_ACC, true>(p, s);
  }
  if (err != hipSuccess) return err;
  {
    LaunchScope scope("gg_gateup_dgrad_f32", s);
    GemmParamsF p = base_f(a);
    p.A = (const float *)a.dh;
    p.B = (const float *)a.w_gu;
    p.C = (float *)a.dx_perm;
    p.N = a.d;
    p.K = 2 * a.F;
    p.lda = 2 * (int64_t)a.F;
    p.ldb = a.d;
    p.ldc = a.d;
    p.strideB = 2 * (int64_t)a.F * a.d;
    p.n_tiles = (a.d + kT - 1) / kT;
    p.total = ragged_total_f(a.R, a.E, p.n_tiles);
    err = run_f32<false, true, F32_STORE, false>(p, s);
  }
  if (err != hipSuccess) return err;
  {
    LaunchScope scope("gg_gateup_wgrad_f32", s);
    GemmParamsF p = base_f(a);
    p.A = (const float *)a.dh;
    p.B = (const float *)a.x_perm;
    p.C = a.dw_gu;
    p.M = 2 * a.F;
    p.N = a.d;
    p.lda = 2 * (int64_t)a.F;
    p.ldb = a.d;
    p.ldc = a.d;
    p.strideC = 2 * (int64_t)a.F * a.d;
    p.m_tiles = (2 * a.F + kT - 1) / kT;
    p.n_tiles = (a.d + kT - 1) / kT;
    p.total = a.E * p.m_tiles * p.n_tiles;
    err = run_f32<true, true, F32_ACC, true>(p, s);
  }
  return err;
}

}  // namespace moe
