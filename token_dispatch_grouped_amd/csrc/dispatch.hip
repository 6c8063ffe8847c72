// Token dispatch and combine: the HBM-bound data movement around the grouped
// expert FFN, forward and backward.
//
// Dispatch moves each token row into the rows of its k experts ("EP token
// dispatch", Add MoE expert parallel training runtime, Major changes); the
// combine returns the weighted expert outputs to full source order (Support
// combined expert and data parallelism in TrainerRank, Desired behavior).
//
// All four kernels move 16-byte chunks: consecutive lanes take consecutive
// chunks of one row, so every row access is a fully coalesced 16 B/lane
// stream. Sums of several rows are formed in fp32 in increasing slot order
// and rounded once. A row index outside [0, T*k) is skipped rather than
// followed, so a corrupted dispatch table cannot write out of bounds.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

// The kernels are instantiated for a maximum slot count KMAX >= k and fully
// unrolled over it, so that all k row indices (and weights) are loaded first
// and all k row accesses of a thread are in flight together. The gathering
// kernels (combine, un-permute backward) read their rows and write their
// outputs with non-temporal accesses: each byte is touched once (measured
// 15-25% faster); the scattering ones keep normal stores, whose rows the
// grouped GEMM reads next (non-temporal stores there measured up to 16%
// slower for the permute in the layer's step, and 2-4% for the combine
// backward).

// A4: x_perm[row_of_slot[t,j]] = x[t]. Each source chunk is read once and
// written k times; a thread copies chunks c and c + nc/2 of one token (nc is
// even: d is a multiple of 64), which keeps twice the stores in flight (one
// chunk per thread, or two adjacent ones, measured slower).
template <typename T, int KMAX>
__global__ __launch_bounds__(256) void permute_kernel(const T *__restrict__ x, const int32_t *__restrict__ ros,
                                                      T *__restrict__ xp, int64_t ntok, int nc, int k) {
  const int64_t nrows = ntok * k;
  constexpr int V = Elem<T>::kVec;
  const int half = nc / 2;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = g / half;
  const int c = (int)(g - t * half);
  if (t >= ntok) return;
  const int64_t ld = (int64_t)nc * V;
  int64_t row[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) row[j] = j < k ? ros[t * k + j] : -1;
  const u32x4_t v0 = ld16(x + t * ld + (int64_t)c * V);
  const u32x4_t v1 = ld16(x + t * ld + (int64_t)(c + half) * V);
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j < k && (uint64_t)row[j] < (uint64_t)nrows) {
      st16(xp + row[j] * ld + (int64_t)c * V, v0);
      st16(xp + row[j] * ld + (int64_t)(c + half) * V, v1);
    }
}

// A7: out[t] = sum_j w[t,j] y[row_of_slot[t,j]].
template <typename T, int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const T *__restrict__ y, const float *__restrict__ tw,
                                                      const int32_t *__restrict__ ros, T *__restrict__ out,
                                                      int64_t ntok, int nc, int k) {
  constexpr int V = Elem<T>::kVec;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = g / nc;
  const int c = (int)(g - t * nc);
  if (t >= ntok) return;
  const int64_t ld = (int64_t)nc * V;
  const int64_t nrows = ntok * k;
  int64_t row[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    row[j] = j < k ? ros[t * k + j] : -1;
    w[j] = j < k ? tw[t * k + j] : 0.f;
  }
  u32x4_t raw[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const bool ok = j < k && (uint64_t)row[j] < (uint64_t)nrows;
    raw[j] = ok ? ld16_nt(y + row[j] * ld + (int64_t)c * V) : u32x4_t{0u, 0u, 0u, 0u};
  }
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    float v[V];
    Elem<T>::unpack(raw[j], v);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = fmaf(w[j], v[i], acc[i]);
  }
  st16_nt(out + t * ld + (int64_t)c * V, Elem<T>::pack(acc));
}

// B1: dy[row] = w[t,j] dout[t];  dtopk_w[t,j] = <dout[t], y[row]>.
// Rows of fewer than 256 chunks: one wavefront per token, a lane taking CPL
// chunks of the row per pass (unrolled, all their loads in flight together;
// the passes repeat until the row is covered). The k dot products are
// reduced across the wavefront.
template <typename T, int CPL, int KMAX>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T *__restrict__ dout, const T *__restrict__ y,
                                                          const float *__restrict__ tw,
                                                          const int32_t *__restrict__ ros, T *__restrict__ dy,
                                                          float *__restrict__ dtw, int64_t ntok, int nc, int k) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const int64_t ld = (int64_t)nc * V;
  const int64_t nrows = ntok * k;
  int64_t row[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    row[j] = j < k ? ros[t * k + j] : -1;
    w[j] = j < k ? tw[t * k + j] : 0.f;
  }
  float dot[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) dot[j] = 0.f;
  for (int c0 = 0; c0 < nc; c0 += CPL * 64) {
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int c = c0 + lane + q * 64;
      if (c >= nc) break;
      float gv[V];
      Elem<T>::unpack(ld16_nt(dout + t * ld + (int64_t)c * V), gv);
      u32x4_t raw[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        const bool ok = j < k && (uint64_t)row[j] < (uint64_t)nrows;
        raw[j] = ok ? ld16_nt(y + row[j] * ld + (int64_t)c * V) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < k && (uint64_t)row[j] < (uint64_t)nrows) {
          float v[V], o[V];
          Elem<T>::unpack(raw[j], v);
#pragma unroll
          for (int i = 0; i < V; ++i) {
            dot[j] = fmaf(gv[i], v[i], dot[j]);
            o[i] = w[j] * gv[i];
          }
          st16(dy + row[j] * ld + (int64_t)c * V, Elem<T>::pack(o));
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      const float d = wave_sum(dot[j]);
      if (lane == 0) dtw[t * k + j] = d;
    }
  }
}

// B1 for rows of 256 to 511 chunks: one workgroup of NT threads per
// token, thread i taking chunks i, i + NT, ...: a token's rows are then read
// and written as NT-chunk runs by the whole workgroup, which streams faster
// than a wavefront walking the row (measured 1% faster at d = 2048). The k
// dot products are reduced in each wavefront, then across the wavefronts in
// a fixed order.
template <typename T, int NT, int KMAX>
__global__ __launch_bounds__(NT) void combine_bwd_wide_kernel(const T *__restrict__ dout, const T *__restrict__ y,
                                                              const float *__restrict__ tw,
                                                              const int32_t *__restrict__ ros, T *__restrict__ dy,
                                                              float *__restrict__ dtw, int64_t ntok, int nc, int k) {
  constexpr int V = Elem<T>::kVec;
  constexpr int NW = NT / 64;
  __shared__ float part[NW][KMAX];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t t = blockIdx.x;
  const int64_t ld = (int64_t)nc * V;
  const int64_t nrows = ntok * k;
  int64_t row[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    row[j] = j < k ? ros[t * k + j] : -1;
    w[j] = j < k ? tw[t * k + j] : 0.f;
  }
  float dot[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) dot[j] = 0.f;
  for (int c = tid; c < nc; c += NT) {
    float gv[V];
    Elem<T>::unpack(ld16_nt(dout + t * ld + (int64_t)c * V), gv);
    u32x4_t raw[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool ok = j < k && (uint64_t)row[j] < (uint64_t)nrows;
      raw[j] = ok ? ld16_nt(y + row[j] * ld + (int64_t)c * V) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k && (uint64_t)row[j] < (uint64_t)nrows) {
        float v[V], o[V];
        Elem<T>::unpack(raw[j], v);
#pragma unroll
        for (int i = 0; i < V; ++i) {
          dot[j] = fmaf(gv[i], v[i], dot[j]);
          o[i] = w[j] * gv[i];
        }
        st16(dy + row[j] * ld + (int64_t)c * V, Elem<T>::pack(o));
      }
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const float d = wave_sum(dot[j]);
    if (lane == 0) part[wv][j] = d;
  }
  __syncthreads();
  if (tid < k) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < NW; ++q) s += part[q][tid];
    dtw[t * k + tid] = s;
  }
}

// B1 for rows of 512 or more chunks (d >= 4096 in bf16): one workgroup of 256
// threads per (token, slot) row, so that each workgroup reads one dout row and one y row,
// writes one dy row and one dot product, with no dependent work across the
// token's k rows (2-3% faster at d = 4096 in the layer's step than one
// workgroup per token walking all k rows; at d = 2048 that form stays, the
// per-row one measured up to 5% slower there). The hardware hands workgroup b to
// XCD b % 8; logical row b is token 8 (q / k) + b % 8, slot q % k with
// q = b / 8, so the k rows of a token run on one XCD and its dout row comes
// from HBM once and from that XCD's L2 for the other slots. The launch holds
// a multiple of 8 workgroups, each stepping through the rows gridDim.x apart.
// A thread takes chunks tid, tid + 256, ... (CPT of them in flight per pass);
// the dot product is reduced per wavefront, then across the four wavefronts
// in a fixed order.
template <typename T, int CPT>
__global__ __launch_bounds__(256) void combine_bwd_row_kernel(const T *__restrict__ dout, const T *__restrict__ y,
                                                              const float *__restrict__ tw,
                                                              const int32_t *__restrict__ ros, T *__restrict__ dy,
                                                              float *__restrict__ dtw, int64_t ntok, int nc, int k,
                                                              int64_t nlogical) {
  constexpr int V = Elem<T>::kVec;
  constexpr int NT = 256, NW = NT / 64;
  __shared__ float part[2][NW];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t ld = (int64_t)nc * V;
  const int64_t nrows = ntok * k;
  int it = 0;
  for (int64_t b = blockIdx.x; b < nlogical; b += gridDim.x, ++it) {
    const int64_t q = b >> 3;
    const int64_t grp = q / k;
    const int64_t t = 8 * grp + (b & 7);
    const int j = (int)(q - grp * k);
    // uniform, and final: the token index only grows along a workgroup's rows
    // (b % 8 is fixed because gridDim.x is a multiple of 8)
    if (t >= ntok) break;
    const int64_t row = ros[t * k + j];
    const float w = tw[t * k + j];
    float dot = 0.f;
    if ((uint64_t)row < (uint64_t)nrows) {
      for (int c0 = 0; c0 < nc; c0 += NT * CPT) {
        u32x4_t g[CPT], yr[CPT];
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
          const int c = c0 + tid + u * NT;
          if (c < nc) {
            g[u] = ld16(dout + t * ld + (int64_t)c * V);  // read again by the token's other slots
            yr[u] = ld16_nt(y + row * ld + (int64_t)c * V);
          }
        }
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
          const int c = c0 + tid + u * NT;
          if (c < nc) {
            float gv[V], v[V], o[V];
            Elem<T>::unpack(g[u], gv);
            Elem<T>::unpack(yr[u], v);
#pragma unroll
            for (int i = 0; i < V; ++i) {
              dot = fmaf(gv[i], v[i], dot);
              o[i] = w * gv[i];
            }
            st16(dy + row * ld + (int64_t)c * V, Elem<T>::pack(o));
          }
        }
      }
    }
    const float ds = wave_sum(dot);
    if (lane == 0) part[it & 1][wv] = ds;
    __syncthreads();  // part[it & 1] is rewritten two rows later, after the next barrier
    if (tid == 0) {
      float s = 0.f;
#pragma unroll
      for (int q2 = 0; q2 < NW; ++q2) s += part[it & 1][q2];
      dtw[t * k + j] = s;
    }
  }
}

// B7: dx[t] = sum_j dx_perm[row_of_slot[t,j]] (+ dx_extra[t]).
template <typename T, int KMAX>
__global__ __launch_bounds__(256) void permute_bwd_kernel(const T *__restrict__ dxp, const int32_t *__restrict__ ros,
                                                          const float *__restrict__ extra, T *__restrict__ dx,
                                                          int64_t ntok, int nc, int k) {
  constexpr int V = Elem<T>::kVec;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = g / nc;
  const int c = (int)(g - t * nc);
  if (t >= ntok) return;
  const int64_t ld = (int64_t)nc * V;
  const int64_t nrows = ntok * k;
  int64_t row[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) row[j] = j < k ? ros[t * k + j] : -1;
  u32x4_t raw[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const bool ok = j < k && (uint64_t)row[j] < (uint64_t)nrows;
    raw[j] = ok ? ld16_nt(dxp + row[j] * ld + (int64_t)c * V) : u32x4_t{0u, 0u, 0u, 0u};
  }
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    float v[V];
    Elem<T>::unpack(raw[j], v);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] += v[i];
  }
  if (extra) {
    const float *e = extra + t * ld + (int64_t)c * V;
#pragma unroll
    for (int i = 0; i < V; i += 4) {
      u32x4_t ev = ld16(e + i);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i + q] += __uint_as_float(ev[q]);
    }
  }
  st16_nt(dx + t * ld + (int64_t)c * V, Elem<T>::pack(acc));
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline unsigned blocks_for(int64_t items) { return (unsigned)((items + 255) / 256); }

// Calls f(std::integral_constant<int, KMAX>) with the smallest KMAX in
// {1, 2, 4, 8, 16} that is >= k.
template <typename F>
static void with_kmax(int k, F &&f) {
  if (k <= 1) f(std::integral_constant<int, 1>{});
  else if (k <= 2) f(std::integral_constant<int, 2>{});
  else if (k <= 4) f(std::integral_constant<int, 4>{});
  else if (k <= 8) f(std::integral_constant<int, 8>{});
  else f(std::integral_constant<int, 16>{});
}

template <typename T>
static void permute_t(const void *x, const int32_t *ros, void *xp, int64_t T_, int d, int k, hipStream_t s) {
  const int nc = d / Elem<T>::kVec;
  with_kmax(k, [&](auto km) {
    constexpr int KM = decltype(km)::value;
    permute_kernel<T, KM><<<blocks_for(T_ * (nc / 2)), 256, 0, s>>>((const T *)x, ros, (T *)xp, T_, nc, k);
  });
}

hipError_t launch_permute(const void *x, const int32_t *row_of_slot, void *x_perm, int64_t T, int d, int k,
                          bool bf16, hipStream_t s) {
  LaunchScope scope("permute", s);
  if (bf16) permute_t<bf16_t>(x, row_of_slot, x_perm, T, d, k, s);
  else permute_t<float>(x, row_of_slot, x_perm, T, d, k, s);
  return hipGetLastError();
}

template <typename T>
static void combine_t(const void *y, const float *tw, const int32_t *ros, void *out, int64_t T_, int d, int k,
                      hipStream_t s) {
  const int nc = d / Elem<T>::kVec;
  with_kmax(k, [&](auto km) {
    constexpr int KM = decltype(km)::value;
    combine_kernel<T, KM><<<blocks_for(T_ * nc), 256, 0, s>>>((const T *)y, tw, ros, (T *)out, T_, nc, k);
  });
}

hipError_t launch_combine(const void *y, const float *topk_w, const int32_t *row_of_slot, void *out, int64_t T,
                          int d, int k, bool bf16, hipStream_t s) {
  LaunchScope scope("combine", s);
  if (bf16) combine_t<bf16_t>(y, topk_w, row_of_slot, out, T, d, k, s);
  else combine_t<float>(y, topk_w, row_of_slot, out, T, d, k, s);
  return hipGetLastError();
}

template <typename T, int CPL>
static void combine_bwd_c(const T *dout, const T *y, const float *tw, const int32_t *ros, T *dy, float *dtw,
                          int64_t ntok, int nc, int k, hipStream_t s) {
  const unsigned grid = (unsigned)((ntok + 3) / 4);
  with_kmax(k, [&](auto km) {
    constexpr int KM = decltype(km)::value;
    combine_bwd_kernel<T, CPL, KM><<<grid, 256, 0, s>>>(dout, y, tw, ros, dy, dtw, ntok, nc, k);
  });
}

template <typename T>
static void combine_bwd_dispatch(const T *dout, const T *y, const float *tw, const int32_t *ros, T *dy,
                                 float *dtw, int64_t ntok, int nc, int k, hipStream_t s) {
  if (nc >= 512) {  // one workgroup per (token, slot) row
    const int64_t nlogical = (ntok + 7) / 8 * 8 * (int64_t)k;
    // one workgroup per row up to 2^20 rows (a multiple of 8); past that the
    // workgroups step over the rest (capping the grid lower measured 3% slower)
    const unsigned grid = (unsigned)std::min<int64_t>(nlogical, (int64_t)1 << 20);
    combine_bwd_row_kernel<T, 2><<<grid, 256, 0, s>>>(dout, y, tw, ros, dy, dtw, ntok, nc, k, nlogical);
    return;
  }
  if (nc >= 256) {  // one workgroup per token
    with_kmax(k, [&](auto km) {
      constexpr int KM = decltype(km)::value;
      combine_bwd_wide_kernel<T, 256, KM><<<dim3((unsigned)ntok), 256, 0, s>>>(dout, y, tw, ros, dy, dtw, ntok, nc, k);
    });
    return;
  }
  const int cpl = (nc + 63) / 64;
  if (cpl <= 1) combine_bwd_c<T, 1>(dout, y, tw, ros, dy, dtw, ntok, nc, k, s);
  else if (cpl <= 2) combine_bwd_c<T, 2>(dout, y, tw, ros, dy, dtw, ntok, nc, k, s);
  else combine_bwd_c<T, 4>(dout, y, tw, ros, dy, dtw, ntok, nc, k, s);
}

hipError_t launch_combine_bwd(const void *dout, const void *y, const float *topk_w, const int32_t *row_of_slot,
                              void *dy, float *dtopk_w, int64_t T, int d, int k, bool bf16, hipStream_t s) {
  LaunchScope scope("combine_bwd", s);
  if (bf16)
    combine_bwd_dispatch<bf16_t>((const bf16_t *)dout, (const bf16_t *)y, topk_w, row_of_slot, (bf16_t *)dy,
                                 dtopk_w, T, d / 8, k, s);
  else
    combine_bwd_dispatch<float>((const float *)dout, (const float *)y, topk_w, row_of_slot, (float *)dy, dtopk_w,
                                T, d / 4, k, s);
  return hipGetLastError();
}

template <typename T>
static void permute_bwd_t(const void *dxp, const int32_t *ros, const float *extra, void *dx, int64_t T_, int d,
                          int k, hipStream_t s) {
  const int nc = d / Elem<T>::kVec;
  with_kmax(k, [&](auto km) {
    constexpr int KM = decltype(km)::value;
    permute_bwd_kernel<T, KM><<<blocks_for(T_ * nc), 256, 0, s>>>((const T *)dxp, ros, extra, (T *)dx, T_, nc, k);
  });
}

hipError_t launch_permute_bwd(const void *dx_perm, const int32_t *row_of_slot, const float *dx_extra, void *dx,
                              int64_t T, int d, int k, bool bf16, hipStream_t s) {
  LaunchScope scope("permute_bwd", s);
  if (bf16) permute_bwd_t<bf16_t>(dx_perm, row_of_slot, dx_extra, dx, T, d, k, s);
  else permute_bwd_t<float>(dx_perm, row_of_slot, dx_extra, dx, T, d, k, s);
  return hipGetLastError();
}

}  // namespace moe
