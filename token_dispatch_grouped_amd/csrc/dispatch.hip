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
#include "common.h"
#include "kernels.h"

namespace moe {

// A4: x_perm[row_of_slot[t,j]] = x[t]. Each source chunk is read once and
// written k times.
template <typename T>
__global__ __launch_bounds__(256) void permute_kernel(const T *__restrict__ x, const int32_t *__restrict__ ros,
                                                      T *__restrict__ xp, int64_t ntok, int nc, int k) {
  const int64_t nrows = ntok * k;
  constexpr int V = Elem<T>::kVec;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = g / nc;
  const int c = (int)(g - t * nc);
  if (t >= ntok) return;
  const int64_t ld = (int64_t)nc * V;
  const u32x4_t v = ld16(x + t * ld + (int64_t)c * V);
  const int32_t *r = ros + t * k;
  for (int j = 0; j < k; ++j) {
    const int64_t row = r[j];
    if ((uint64_t)row < (uint64_t)nrows) st16(xp + row * ld + (int64_t)c * V, v);
  }
}

// A7: out[t] = sum_j w[t,j] y[row_of_slot[t,j]].
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T *__restrict__ y, const float *__restrict__ tw,
                                                      const int32_t *__restrict__ ros, T *__restrict__ out,
                                                      int64_t ntok, int nc, int k) {
  constexpr int V = Elem<T>::kVec;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = g / nc;
  const int c = (int)(g - t * nc);
  if (t >= ntok) return;
  const int64_t ld = (int64_t)nc * V;
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  for (int j = 0; j < k; ++j) {
    const float w = tw[t * k + j];
    const int64_t row = ros[t * k + j];
    if ((uint64_t)row >= (uint64_t)(ntok * k)) continue;
    float v[V];
    Elem<T>::unpack(ld16(y + row * ld + (int64_t)c * V), v);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = fmaf(w, v[i], acc[i]);
  }
  st16(out + t * ld + (int64_t)c * V, Elem<T>::pack(acc));
}

// B1: dy[row] = w[t,j] dout[t];  dtopk_w[t,j] = <dout[t], y[row]>.
// One wavefront per token: each lane holds CPL chunks of dout, the k dot
// products are reduced across the wavefront.
template <typename T, int CPL>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T *__restrict__ dout, const T *__restrict__ y,
                                                          const float *__restrict__ tw,
                                                          const int32_t *__restrict__ ros, T *__restrict__ dy,
                                                          float *__restrict__ dtw, int64_t ntok, int nc, int k) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const int64_t ld = (int64_t)nc * V;
  float g[CPL][V];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    const int c = lane + q * 64;
    if (c < nc) {
      Elem<T>::unpack(ld16(dout + t * ld + (int64_t)c * V), g[q]);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) g[q][i] = 0.f;
    }
  }
  for (int j = 0; j < k; ++j) {
    const float w = tw[t * k + j];
    const int64_t row = ros[t * k + j];
    const bool in = (uint64_t)row < (uint64_t)(ntok * k);
    float dot = 0.f;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int c = lane + q * 64;
      if (c < nc && in) {
        float v[V], o[V];
        Elem<T>::unpack(ld16(y + row * ld + (int64_t)c * V), v);
#pragma unroll
        for (int i = 0; i < V; ++i) {
          dot = fmaf(g[q][i], v[i], dot);
          o[i] = w * g[q][i];
        }
        st16(dy + row * ld + (int64_t)c * V, Elem<T>::pack(o));
      }
    }
    dot = wave_sum(dot);
    if (lane == 0) dtw[t * k + j] = dot;
  }
}

// B7: dx[t] = sum_j dx_perm[row_of_slot[t,j]] (+ dx_extra[t]).
template <typename T>
__global__ __launch_bounds__(256) void permute_bwd_kernel(const T *__restrict__ dxp, const int32_t *__restrict__ ros,
                                                          const float *__restrict__ extra, T *__restrict__ dx,
                                                          int64_t ntok, int nc, int k) {
  constexpr int V = Elem<T>::kVec;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = g / nc;
  const int c = (int)(g - t * nc);
  if (t >= ntok) return;
  const int64_t ld = (int64_t)nc * V;
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int64_t row = ros[t * k + j];
    if ((uint64_t)row >= (uint64_t)(ntok * k)) continue;
    float v[V];
    Elem<T>::unpack(ld16(dxp + row * ld + (int64_t)c * V), v);
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
  st16(dx + t * ld + (int64_t)c * V, Elem<T>::pack(acc));
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline unsigned blocks_for(int64_t items) { return (unsigned)((items + 255) / 256); }

hipError_t launch_permute(const void *x, const int32_t *row_of_slot, void *x_perm, int64_t T, int d, int k,
                          bool bf16, hipStream_t s) {
  LaunchScope scope("permute", s);
  if (bf16) {
    const int nc = d / 8;
    permute_kernel<bf16_t><<<blocks_for(T * nc), 256, 0, s>>>((const bf16_t *)x, row_of_slot, (bf16_t *)x_perm, T,
                                                              nc, k);
  } else {
    const int nc = d / 4;
    permute_kernel<float><<<blocks_for(T * nc), 256, 0, s>>>((const float *)x, row_of_slot, (float *)x_perm, T, nc,
                                                             k);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const void *y, const float *topk_w, const int32_t *row_of_slot, void *out, int64_t T,
                          int d, int k, bool bf16, hipStream_t s) {
  LaunchScope scope("combine", s);
  if (bf16) {
    const int nc = d / 8;
    combine_kernel<bf16_t><<<blocks_for(T * nc), 256, 0, s>>>((const bf16_t *)y, topk_w, row_of_slot,
                                                              (bf16_t *)out, T, nc, k);
  } else {
    const int nc = d / 4;
    combine_kernel<float><<<blocks_for(T * nc), 256, 0, s>>>((const float *)y, topk_w, row_of_slot, (float *)out,
                                                             T, nc, k);
  }
  return hipGetLastError();
}

template <typename T>
static void combine_bwd_dispatch(const T *dout, const T *y, const float *tw, const int32_t *ros, T *dy,
                                 float *dtw, int64_t ntok, int nc, int k, hipStream_t s) {
  const unsigned grid = (unsigned)((ntok + 3) / 4);
  const int cpl = (nc + 63) / 64;
  if (cpl <= 1)
    combine_bwd_kernel<T, 1><<<grid, 256, 0, s>>>(dout, y, tw, ros, dy, dtw, ntok, nc, k);
  else if (cpl <= 2)
    combine_bwd_kernel<T, 2><<<grid, 256, 0, s>>>(dout, y, tw, ros, dy, dtw, ntok, nc, k);
  else if (cpl <= 4)
    combine_bwd_kernel<T, 4><<<grid, 256, 0, s>>>(dout, y, tw, ros, dy, dtw, ntok, nc, k);
  else if (cpl <= 8)
    combine_bwd_kernel<T, 8><<<grid, 256, 0, s>>>(dout, y, tw, ros, dy, dtw, ntok, nc, k);
  else if (cpl <= 16)
    combine_bwd_kernel<T, 16><<<grid, 256, 0, s>>>(dout, y, tw, ros, dy, dtw, ntok, nc, k);
  else
    combine_bwd_kernel<T, 32><<<grid, 256, 0, s>>>(dout, y, tw, ros, dy, dtw, ntok, nc, k);
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

hipError_t launch_permute_bwd(const void *dx_perm, const int32_t *row_of_slot, const float *dx_extra, void *dx,
                              int64_t T, int d, int k, bool bf16, hipStream_t s) {
  LaunchScope scope("permute_bwd", s);
  if (bf16) {
    const int nc = d / 8;
    permute_bwd_kernel<bf16_t><<<blocks_for(T * nc), 256, 0, s>>>((const bf16_t *)dx_perm, row_of_slot, dx_extra,
                                                                  (bf16_t *)dx, T, nc, k);
  } else {
    const int nc = d / 4;
    permute_bwd_kernel<float><<<blocks_for(T * nc), 256, 0, s>>>((const float *)dx_perm, row_of_slot, dx_extra,
                                                                 (float *)dx, T, nc, k);
  }
  return hipGetLastError();
}

}  // namespace moe
