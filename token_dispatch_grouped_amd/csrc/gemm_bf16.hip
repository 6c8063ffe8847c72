// Grouped expert GEMMs in bf16 on the gfx950 matrix cores ("grouped expert
// compute", Add MoE expert parallel training runtime, Major changes).
//
// One kernel template covers the six products of the SwiGLU expert FFN,
// forward and backward. For expert e it computes
//     C_e[m, n] = sum_k A_e(m, k) * B_e(n, k)
// where each operand is read either k-contiguous ("N" layout, row-major
// [rows, K]) or transposed (row-major [K, rows]):
//   gate/up fwd   H  = X W_gu^T      A = x_perm [R,d]  B = W_gu[e] [2F,d]   ragged M
//   down fwd      Y  = A W_down^T    A = a [R,F]       B = W_down[e] [d,F]  ragged M
//   down dgrad    dA = dY W_down     A = dy [R,d]      B^T = W_down[e]      ragged M
//   gate/up dgrad dX = dH W_gu       A = dh [R,2F]     B^T = W_gu[e]        ragged M
//   down wgrad    dW_down += dY^T a  A^T = dy, B^T = a                      ragged K
//   gate/up wgrad dW_gu  += dH^T X   A^T = dh, B^T = x_perm                 ragged K
// "Ragged" is the per-expert row count M_e = offsets[e+1] - offsets[e],
// which the host never reads: workgroups find their expert and tile from
// `offsets` on the device, so an expert with no rows gets no tile at all and
// any M_e (0 included) needs no padding.
//
// Tiling: a 256-thread workgroup (4 wavefronts) computes a BM x BN tile with
// BK = 64 deep k-steps, double-buffered in LDS. Both operands are stored in
// LDS k-contiguous, in 16-byte chunks with an XOR swizzle so that the
// fragment reads of v_mfma_f32_32x32x16_bf16 and the tile writes are free of
// bank conflicts. Transposed operands are turned k-contiguous on the way in:
// each thread loads an 8(k) x 8 block with eight 16-byte loads and transposes
// it in registers. Accumulation is fp32; the epilogue rounds once.
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

enum { EPI_STORE = 0, EPI_SWIGLU_FWD = 1, EPI_SWIGLU_BWD = 2, EPI_ACC_F32 = 3 };

struct GemmParams {
  const bf16_t *A;
  const bf16_t *B;
  void *C;                // bf16 output, or fp32 accumulator (EPI_ACC_F32)
  bf16_t *C2;             // EPI_SWIGLU_FWD: the activation a
  const bf16_t *H;        // EPI_SWIGLU_BWD: saved h
  const int32_t *offsets;
  int E;
  int M;                  // ragged K: rows of C
  int N;                  // columns of C (EPI_SWIGLU_FWD: F, the gate half)
  int K;                  // ragged M: reduction length
  int64_t lda, ldb, ldc;
  int64_t strideB;        // ragged M: per-expert stride of B
  int64_t strideC;        // ragged K: per-expert stride of C
  int F;
  int n_tiles, m_tiles;
  int total;              // logical workgroups
};

constexpr int kBK = 64;

MOE_DEVICE int swz(int row) { return (row ^ (row >> 3)) & 7; }

// Combine two bf16 lanes: element `j` of dword words a and b.
MOE_DEVICE uint32_t pick_pair(uint32_t a, uint32_t b, int odd) {
  return odd ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

template <int BM, int BN, int WM, int WN, bool AT, bool BT, int EPI, bool RAGGED_K>
__global__ __launch_bounds__(256, 2) void gg_bf16_kernel(GemmParams p) {
  constexpr int WAVES_N = BN / WN;
  constexpr int WAVES_M = BM / WM;
  static_assert(WAVES_M * WAVES_N == 4, "4 wavefronts per workgroup");
  constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(EPI != EPI_SWIGLU_FWD || (FN % 2) == 0, "gate/up pairs need an even fragment count");
  // 16-byte chunks per operand tile
  constexpr int A_CHUNKS = BM * kBK / 8;
  constexpr int B_CHUNKS = BN * kBK / 8;
  // per-thread staging (N layout: chunks; transposed layout: 8x8 blocks)
  constexpr int A_NL = AT ? 0 : A_CHUNKS / 256;
  constexpr int B_NL = BT ? 0 : B_CHUNKS / 256;
  constexpr int A_SUB = AT ? BM * kBK / 64 : 0;  // 8x8 sub-blocks
  constexpr int B_SUB = BT ? BN * kBK / 64 : 0;
  static_assert(AT || A_CHUNKS % 256 == 0, "tile/thread mismatch");
  static_assert(BT || B_CHUNKS % 256 == 0, "tile/thread mismatch");
  // transposed operands: when both are transposed, threads 0..127 load A and
  // 128..255 load B; otherwise all threads share the one transposed operand.
  constexpr bool SPLIT_T = AT && BT;
  constexpr int T_THREADS = SPLIT_T ? 128 : 256;
  constexpr int A_TR = AT ? (A_SUB + T_THREADS - 1) / T_THREADS : 0;
  constexpr int B_TR = BT ? (B_SUB + T_THREADS - 1) / T_THREADS : 0;

  __shared__ u32x4_t lds[2][A_CHUNKS + B_CHUNKS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  if (bid >= p.total) return;

  int e, m0, n_tile, m_valid, kdim;
  int64_t crow0;  // ragged M: first C row of the tile
  const bf16_t *Ab;
  const bf16_t *Bb;
  if (!RAGGED_K) {
    n_tile = bid % p.n_tiles;
    const int mslot = bid / p.n_tiles;
    int mt;
    if (!find_m_tile<BM>(p.offsets, p.E, mslot, e, mt)) return;
    const int row0 = p.offsets[e];
    const int me = p.offsets[e + 1] - row0;
    m0 = mt * BM;
    m_valid = min(BM, me - m0);
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
    if (kdim <= 0) return;  // empty expert: dW stays bit-identical
    m0 = mt * BM;
    m_valid = min(BM, p.M - m0);
    crow0 = 0;
    Ab = p.A + (int64_t)row0 * p.lda;
    Bb = p.B + (int64_t)row0 * p.ldb;
  }

  // Global row (or column, for transposed B) of B-tile row r.
  auto b_row = [&](int r) -> int {
    if (EPI == EPI_SWIGLU_FWD) {
      const int wcol = r / WN, q = r % WN;
      const int g = n_tile * (BN / 2) + wcol * (WN / 2) + (q % (WN / 2));
      return g < p.N ? (q < WN / 2 ? g : p.F + g) : -1;
    } else {
      const int n = n_tile * BN + r;
      return n < p.N ? n : -1;
    }
  };

  u32x4_t ra[A_NL > 0 ? A_NL : 1];
  u32x4_t rb[B_NL > 0 ? B_NL : 1];
  u32x4_t ta[A_TR > 0 ? A_TR : 1][8];
  u32x4_t tb[B_TR > 0 ? B_TR : 1][8];

  auto load_tiles = [&](int k0) {
    // --- A ---
    if (!AT) {
#pragma unroll
      for (int i = 0; i < A_NL; ++i) {
        const int c = i * 256 + tid;
        const int r = c >> 3, ch = c & 7;
        const int rr = r < m_valid ? r : m_valid - 1;
        ra[i] = ld16(Ab + (int64_t)rr * p.lda + k0 + ch * 8);
      }
    } else {
      const int t2 = SPLIT_T ? tid : tid;
#pragma unroll
      for (int i = 0; i < A_TR; ++i) {
        const int sidx = i * T_THREADS + t2;
        const int xb = sidx % (BM / 8), kb = sidx / (BM / 8);
        const bool on = (!SPLIT_T || tid < 128) && sidx < A_SUB && (xb * 8 < m_valid);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int kk = k0 + kb * 8 + q;
          if (on && kk < kdim)
            ta[i][q] = ld16(Ab + (int64_t)kk * p.lda + m0 + xb * 8);
          else
            ta[i][q] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
    // --- B ---
    if (!BT) {
#pragma unroll
      for (int i = 0; i < B_NL; ++i) {
        const int c = i * 256 + tid;
        const int r = c >> 3, ch = c & 7;
        const int g = b_row(r);
        if (g >= 0)
          rb[i] = ld16(Bb + (int64_t)g * p.ldb + k0 + ch * 8);
        else
          rb[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
    } else {
      const int t2 = SPLIT_T ? tid - 128 : tid;
#pragma unroll
      for (int i = 0; i < B_TR; ++i) {
        const int sidx = i * T_THREADS + t2;
        const int xb = sidx % (BN / 8), kb = sidx / (BN / 8);
        const int n = n_tile * BN + xb * 8;
        const bool on = (!SPLIT_T || tid >= 128) && sidx >= 0 && sidx < B_SUB && n < p.N;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int kk = k0 + kb * 8 + q;
          if (on && kk < kdim)
            tb[i][q] = ld16(Bb + (int64_t)kk * p.ldb + n);
          else
            tb[i][q] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  auto store_tiles = [&](int buf) {
    u32x4_t *As = lds[buf];
    u32x4_t *Bs = lds[buf] + A_CHUNKS;
    if (!AT) {
#pragma unroll
      for (int i = 0; i < A_NL; ++i) {
        const int c = i * 256 + tid;
        const int r = c >> 3, ch = c & 7;
        As[r * 8 + (ch ^ swz(r))] = ra[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < A_TR; ++i) {
        const int sidx = i * T_THREADS + (SPLIT_T ? tid : tid);
        const bool on = (!SPLIT_T || tid < 128) && sidx < A_SUB;
        if (on) {
          const int xb = sidx % (BM / 8), kb = sidx / (BM / 8);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            u32x4_t o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = pick_pair(ta[i][2 * q][j >> 1], ta[i][2 * q + 1][j >> 1], j & 1);
            const int r = xb * 8 + j;
            As[r * 8 + (kb ^ swz(r))] = o;
          }
        }
      }
    }
    if (!BT) {
#pragma unroll
      for (int i = 0; i < B_NL; ++i) {
        const int c = i * 256 + tid;
        const int r = c >> 3, ch = c & 7;
        Bs[r * 8 + (ch ^ swz(r))] = rb[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_TR; ++i) {
        const int sidx = i * T_THREADS + (SPLIT_T ? tid - 128 : tid);
        const bool on = (!SPLIT_T || tid >= 128) && sidx >= 0 && sidx < B_SUB;
        if (on) {
          const int xb = sidx % (BN / 8), kb = sidx / (BN / 8);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            u32x4_t o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = pick_pair(tb[i][2 * q][j >> 1], tb[i][2 * q + 1][j >> 1], j & 1);
            const int r = xb * 8 + j;
            Bs[r * 8 + (kb ^ swz(r))] = o;
          }
        }
      }
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = (kdim + kBK - 1) / kBK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();

  const int l32 = lane & 31;
  const int lhi = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tiles((kt + 1) * kBK);
    const u32x4_t *As = lds[cur];
    const u32x4_t *Bs = lds[cur] + A_CHUNKS;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int ch = ks * 2 + lhi;
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WM + i * 32 + l32;
        af[i] = __builtin_bit_cast(bf16x8_t, As[r * 8 + (ch ^ swz(r))]);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * WN + j * 32 + l32;
        bfr[j] = __builtin_bit_cast(bf16x8_t, Bs[r * 8 + (ch ^ swz(r))]);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tiles(cur ^ 1);
    __syncthreads();
  }

  // ---------------- epilogue ----------------
  // acc[i][j][v] sits at tile row wm*WM + i*32 + 8*(v/4) + 4*lhi + (v%4),
  // tile column wn*WN + j*32 + l32.
  if (EPI == EPI_SWIGLU_FWD) {
    bf16_t *H = (bf16_t *)p.C;
    bf16_t *Aout = p.C2;
#pragma unroll
    for (int j = 0; j < FN / 2; ++j) {
      const int g = n_tile * (BN / 2) + wn * (WN / 2) + j * 32 + l32;
      if (g >= p.N) continue;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * WM + i * 32 + 8 * (v >> 2) + 4 * lhi + (v & 3);
          if (r < m_valid) {
            const float gt = acc[i][j][v];
            const float up = acc[i][j + FN / 2][v];
            const int64_t row = crow0 + r;
            H[row * p.ldc + g] = f2bf(gt);
            H[row * p.ldc + p.F + g] = f2bf(up);
            Aout[row * p.F + g] = f2bf(silu_f(gt) * up);
          }
        }
    }
  } else if (EPI == EPI_SWIGLU_BWD) {
    bf16_t *dH = (bf16_t *)p.C;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n_tile * BN + wn * WN + j * 32 + l32;
      if (n >= p.N) continue;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * WM + i * 32 + 8 * (v >> 2) + 4 * lhi + (v & 3);
          if (r < m_valid) {
            const int64_t row = crow0 + r;
            const float da = acc[i][j][v];
            const float hg = bf2f(p.H[row * p.ldc + n]);
            const float hu = bf2f(p.H[row * p.ldc + p.F + n]);
            const float sg = sigmoid_f(hg);
            dH[row * p.ldc + n] = f2bf(da * hu * sg * (1.f + hg * (1.f - sg)));
            dH[row * p.ldc + p.F + n] = f2bf(da * hg * sg);
          }
        }
    }
  } else if (EPI == EPI_STORE) {
    bf16_t *C = (bf16_t *)p.C;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n_tile * BN + wn * WN + j * 32 + l32;
      if (n >= p.N) continue;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * WM + i * 32 + 8 * (v >> 2) + 4 * lhi + (v & 3);
          if (r < m_valid) C[(crow0 + r) * p.ldc + n] = f2bf(acc[i][j][v]);
        }
    }
  } else {  // EPI_ACC_F32
    float *C = (float *)p.C + (int64_t)e * p.strideC;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n_tile * BN + wn * WN + j * 32 + l32;
      if (n >= p.N) continue;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * WM + i * 32 + 8 * (v >> 2) + 4 * lhi + (v & 3);
          if (r < m_valid) {
            float *dst = C + (int64_t)(m0 + r) * p.ldc + n;
            *dst = *dst + acc[i][j][v];
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, bool AT, bool BT, int EPI, bool RAGGED_K>
static hipError_t run_gemm(GemmParams p, hipStream_t s) {
  if (p.total <= 0) return hipSuccess;
  const int grid = (p.total + 7) / 8 * 8;
  gg_bf16_kernel<BM, BN, WM, WN, AT, BT, EPI, RAGGED_K><<<dim3((unsigned)grid), 256, 0, s>>>(p);
  return hipGetLastError();
}

static GemmParams base_params(const GroupedFfnArgs &a) {
  GemmParams p{};
  p.offsets = a.offsets;
  p.E = a.E;
  p.F = a.F;
  return p;
}

// Ragged-M grid: an upper bound of the number of BM-row tiles over all
// experts (sum of ceil(M_e/BM) <= R/BM + E), times the column tiles.
static int ragged_m_total(int64_t R, int E, int BM, int n_tiles) {
  return (int)((R / BM + E) * (int64_t)n_tiles);
}

constexpr int kBM = kGemmBM, kBN = kGemmBN, kWM = 64, kWN = 64;

hipError_t launch_ffn_fwd_bf16(const GroupedFfnArgs &a, hipStream_t s) {
  hipError_t err;
  {
    LaunchScope scope("gg_gateup_fwd", s);
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
    p.n_tiles = (a.F + kBN / 2 - 1) / (kBN / 2);
    p.total = ragged_m_total(a.R, a.E, kBM, p.n_tiles);
    err = run_gemm<kBM, kBN, kWM, kWN, false, false, EPI_SWIGLU_FWD, false>(p, s);
  }
  if (err != hipSuccess) return err;
  {
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
    p.n_tiles = (a.d + kBN - 1) / kBN;
    p.total = ragged_m_total(a.R, a.E, kBM, p.n_tiles);
    err = run_gemm<kBM, kBN, kWM, kWN, false, false, EPI_STORE, false>(p, s);
  }
  return err;
}

hipError_t launch_ffn_bwd_bf16(const GroupedFfnArgs &a, hipStream_t s) {
  hipError_t err;
  {  // B3: dA = dY W_down[e], SwiGLU backward in the epilogue -> dH
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
    p.n_tiles = (a.F + kBN - 1) / kBN;
    p.total = ragged_m_total(a.R, a.E, kBM, p.n_tiles);
    err = run_gemm<kBM, kBN, kWM, kWN, false, true, EPI_SWIGLU_BWD, false>(p, s);
  }
  if (err != hipSuccess) return err;
  {  // B4: dW_down[e] += dY_e^T a_e
    LaunchScope scope("gg_down_wgrad", s);
    GemmParams p = base_params(a);
    p.A = (const bf16_t *)a.dy;
    p.B = (const bf16_t *)a.a;
    p.C = a.dw_down;
    p.M = a.d;
    p.N = a.F;
    p.lda = a.d;
    p.ldb = a.F;
    p.ldc = a.F;
    p.strideC = (int64_t)a.d * a.F;
    p.m_tiles = (a.d + kBM - 1) / kBM;
    p.n_tiles = (a.F + kBN - 1) / kBN;
    p.total = a.E * p.m_tiles * p.n_tiles;
    err = run_gemm<kBM, kBN, kWM, kWN, true, true, EPI_ACC_F32, true>(p, s);
  }
  if (err != hipSuccess) return err;
  {  // B5: dX_perm = dH W_gu[e]
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
    p.n_tiles = (a.d + kBN - 1) / kBN;
    p.total = ragged_m_total(a.R, a.E, kBM, p.n_tiles);
    err = run_gemm<kBM, kBN, kWM, kWN, false, true, EPI_STORE, false>(p, s);
  }
  if (err != hipSuccess) return err;
  {  // B6: dW_gu[e] += dH^T X_e
    LaunchScope scope("gg_gateup_wgrad", s);
    GemmParams p = base_params(a);
    p.A = (const bf16_t *)a.dh;
    p.B = (const bf16_t *)a.x_perm;
    p.C = a.dw_gu;
    p.M = 2 * a.F;
    p.N = a.d;
    p.lda = 2 * (int64_t)a.F;
    p.ldb = a.d;
    p.ldc = a.d;
    p.strideC = 2 * (int64_t)a.F * a.d;
    p.m_tiles = (2 * a.F + kBM - 1) / kBM;
    p.n_tiles = (a.d + kBN - 1) / kBN;
    p.total = a.E * p.m_tiles * p.n_tiles;
    err = run_gemm<kBM, kBN, kWM, kWN, true, true, EPI_ACC_F32, true>(p, s);
  }
  return err;
}

}  // namespace moe
