// Routing kernels: router logits, top-k softmax selection with a
// deterministic stable counting sort into expert-contiguous rows, and the
// routing backward.
//
// The pages name the step ("EP token dispatch", Add MoE expert parallel
// training runtime, Major changes) and require that any per-expert row count,
// zero included, works without padding and that outputs return in full
// source order (Support combined expert and data parallelism in TrainerRank,
// Desired behavior). The rule implemented: the k largest logits of a token,
// descending, equal logits to the lower expert id; weights are the softmax
// probabilities of the selected experts (optionally renormalised); rows of
// one expert follow ascending source token.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// A1: logits = x w_router^T + bias. One wavefront per token; lanes split the
// hidden dimension in 16-byte chunks, experts are taken 16 at a time and each
// partial dot product is reduced across the wavefront.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void router_logits_kernel(const T *__restrict__ x, const T *__restrict__ wr,
                                                            const float *__restrict__ bias,
                                                            float *__restrict__ logits, int64_t ntok, int d,
                                                            int E) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const T *xr = x + t * d;
  const int nchunk = d / V;
  for (int e0 = 0; e0 < E; e0 += 16) {
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    for (int c = lane; c < nchunk; c += 64) {
      float xv[V];
      Elem<T>::unpack(ld16(xr + (size_t)c * V), xv);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (e0 + i < E) {
          float wv[V];
          Elem<T>::unpack(ld16(wr + (size_t)(e0 + i) * d + (size_t)c * V), wv);
#pragma unroll
          for (int q = 0; q < V; ++q) acc[i] = fmaf(xv[q], wv[q], acc[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (e0 + i < E) {
        float s = wave_sum(acc[i]);
        if (lane == 0) logits[t * E + e0 + i] = s + (bias ? bias[e0 + i] : 0.f);
      }
    }
  }
}

// Order-preserving map of fp32 onto uint32: larger value -> larger key, NaN
// below everything (key 0), -0.0 equal to +0.0.
MOE_DEVICE uint32_t order_key(float f) {
  if (f != f) return 0u;
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Visit row[0..E) in ascending order, f(e, value). With E % 4 == 0 (rows
// then 16-byte aligned) the row is read 16 values at a time by four 16-byte
// loads issued together, so that a thread waits for one round trip per 16
// values instead of one per value.
template <typename F>
MOE_DEVICE void for_row(const float *__restrict__ row, int E, F f) {
  int e0 = 0;
  if ((E & 3) == 0) {
    for (; e0 + 16 <= E; e0 += 16) {
      float4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const float4 *>(row + e0 + 4 * i);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f(e0 + 4 * i, v[i].x);
        f(e0 + 4 * i + 1, v[i].y);
        f(e0 + 4 * i + 2, v[i].z);
        f(e0 + 4 * i + 3, v[i].w);
      }
    }
    for (; e0 < E; e0 += 4) {
      const float4 v = *reinterpret_cast<const float4 *>(row + e0);
      f(e0, v.x);
      f(e0 + 1, v.y);
      f(e0 + 2, v.z);
      f(e0 + 3, v.w);
    }
    return;
  }
  for (; e0 < E; ++e0) f(e0, row[e0]);
}

// ---------------------------------------------------------------------------
// A2 + first half of A3: per token top-k and weights; per workgroup the
// stable rank of each (token, slot) among the workgroup's slots of the same
// expert, and the workgroup's expert histogram.
//
// One thread per token, kRouteTokensPerBlock tokens per workgroup (one
// wavefront: 512 workgroups at 32k tokens, so every CU gets work). Top-k keeps
// a descending list of 64-bit composite keys (logit key, then inverted id so
// that the lower id wins a tie). A token selects an expert at most once, so
// the rank of slot (t, j) among the workgroup's slots of expert e is the
// number of earlier tokens of the workgroup that selected e. Each wavefront
// builds in LDS, per expert, the 64-bit mask of its lanes that selected it
// (bitwise OR, whose result does not depend on the order of the updates);
// the rank is the population count of the masks of earlier wavefronts plus
// that of the own mask below the lane. No atomic decides any order.
// ---------------------------------------------------------------------------
template <int KMAX>
__global__ __launch_bounds__(kRouteTokensPerBlock) void route_topk_kernel(const float *__restrict__ logits,
                                                         int32_t *__restrict__ topk_idx,
                                                         float *__restrict__ topk_w,
                                                         int32_t *__restrict__ local_rank,
                                                         int32_t *__restrict__ blk_cnt, int64_t ntok, int E,
                                                         int k, int renorm) {
  constexpr int NT = kRouteTokensPerBlock;
  constexpr int NW = NT / 64;
  static_assert(NW * 64 == NT, "whole wavefronts per workgroup");
  __shared__ unsigned long long s_mask[NW][256];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int64_t t = (int64_t)blockIdx.x * NT + tid;
  const bool valid = t < ntok;

  for (int i = tid; i < NW * 256; i += NT) (&s_mask[0][0])[i] = 0ull;

  uint64_t list[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) list[i] = 0ull;
  int ids[KMAX];
  float w[KMAX];
  if (valid) {
    const float *row = logits + t * E;
    for_row(row, E, [&](int e, float l) {
      uint64_t c = ((uint64_t)order_key(l) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
      if (c > list[KMAX - 1]) {
        // insert into the descending list: entries above c stay, c takes the
        // first place it beats, the entries below shift down one place
        bool g[KMAX];
#pragma unroll
        for (int i = 0; i < KMAX; ++i) g[i] = c > list[i];
#pragma unroll
        for (int i = KMAX - 1; i > 0; --i) list[i] = g[i - 1] ? list[i - 1] : (g[i] ? c : list[i]);
        list[0] = g[0] ? c : list[0];
      }
    });
#pragma unroll
    for (int i = 0; i < KMAX; ++i) ids[i] = (int)(0xffffffffu - (uint32_t)(list[i] & 0xffffffffu));
    // softmax over the whole row; the first selected logit is the maximum
    const float m = row[ids[0]];
    float sum = 0.f;
    for_row(row, E, [&](int, float l) { sum += (l == l) ? expf(l - m) : 0.f; });
    float wsum = 0.f;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      float l = row[(unsigned)ids[i] < (unsigned)E ? ids[i] : 0];
      w[i] = (i < k && l == l) ? expf(l - m) / sum : 0.f;
      if (i < k) wsum += w[i];
    }
    if (renorm) {
#pragma unroll
      for (int i = 0; i < KMAX; ++i) w[i] = w[i] / wsum;
    }
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (i < k) {
        topk_idx[t * k + i] = ids[i];
        topk_w[t * k + i] = w[i];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < KMAX; ++i) ids[i] = 0;
  }
  __syncthreads();  // masks cleared
  if (valid) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) atomicOr(&s_mask[wave][ids[j]], 1ull << lane);
  }
  __syncthreads();
  if (valid) {
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        int pre = __popcll(s_mask[wave][ids[j]] & below);
        for (int w2 = 0; w2 < wave; ++w2) pre += __popcll(s_mask[w2][ids[j]]);
        local_rank[t * k + j] = pre;
      }
    }
  }
  for (int e = tid; e < E; e += NT) {
    int c = 0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) c += __popcll(s_mask[w2][e]);
    blk_cnt[(int64_t)blockIdx.x * E + e] = c;
  }
}

// Block-wide exclusive scan of one int per thread (256 threads); returns the
// exclusive prefix and writes the block total to *total.
MOE_DEVICE int block_exclusive_scan_256(int v, int *s_tmp, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = wave_inclusive_scan(v);
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  int wpre = 0, all = 0;
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    int tv = s_tmp[w2];
    if (w2 < wave) wpre += tv;
    all += tv;
  }
  __syncthreads();
  *total = all;
  return wpre + inc - v;
}

// Second half of A3, step 1: per expert, exclusive scan of the workgroup
// histograms over workgroups (in place), and the expert's total row count.
__global__ __launch_bounds__(256) void route_scan_kernel(int32_t *__restrict__ blk_cnt,
                                                         int32_t *__restrict__ counts, int64_t nblk, int E) {
  __shared__ int s_tmp[4];
  const int e = blockIdx.x;
  int carry = 0;
  for (int64_t b0 = 0; b0 < nblk; b0 += 256) {
    const int64_t b = b0 + threadIdx.x;
    int v = b < nblk ? blk_cnt[b * E + e] : 0;
    int tot;
    int ex = block_exclusive_scan_256(v, s_tmp, &tot);
    if (b < nblk) blk_cnt[b * E + e] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

// Second half of A3, step 2: offsets, final rows and the inverse map.
// row = offsets[e] + (rows of e in earlier workgroups) + (rank in workgroup).
__global__ __launch_bounds__(256) void route_rows_kernel(const int32_t *__restrict__ topk_idx,
                                                         const int32_t *__restrict__ counts,
                                                         const int32_t *__restrict__ blk_cnt,
                                                         int32_t *__restrict__ row_of_slot,
                                                         int32_t *__restrict__ src_of_row,
                                                         int32_t *__restrict__ offsets, int64_t nslot, int E,
                                                         int k) {
  __shared__ int s_off[257];
  __shared__ int s_tmp[4];
  const int tid = threadIdx.x;
  int v = tid < E ? counts[tid] : 0;
  int tot;
  int ex = block_exclusive_scan_256(v, s_tmp, &tot);
  s_off[tid] = ex;
  if (tid == 0) s_off[256] = tot;
  __syncthreads();
  if (blockIdx.x == 0) {
    if (tid < E) offsets[tid] = ex;
    if (tid == 0) offsets[E] = tot;
  }
  const int64_t s = (int64_t)blockIdx.x * 256 + tid;
  if (s >= nslot) return;
  const int e = topk_idx[s];
  const int64_t t = s / k;
  const int64_t b = t / kRouteTokensPerBlock;
  const int row = s_off[e] + blk_cnt[b * E + e] + row_of_slot[s];
  row_of_slot[s] = row;
  if ((uint64_t)row < (uint64_t)nslot) src_of_row[row] = (int32_t)s;
}

// ---------------------------------------------------------------------------
// B2: dlogits from dtopk_w. One thread per token.
// ---------------------------------------------------------------------------
constexpr int kRouteBwdThreads = 64;  // one wavefront per workgroup: 512 workgroups at 32k tokens

template <int KMAX>
__global__ __launch_bounds__(kRouteBwdThreads) void route_bwd_kernel(const float *__restrict__ dtopk_w,
                                                        const float *__restrict__ logits,
                                                        const int32_t *__restrict__ topk_idx,
                                                        const float *__restrict__ topk_w,
                                                        float *__restrict__ dlogits, int64_t ntok, int E, int k,
                                                        int renorm, int accumulate) {
  const int64_t t = (int64_t)blockIdx.x * kRouteBwdThreads + threadIdx.x;
  if (t >= ntok) return;
  const float *row = logits + t * E;
  float *drow = dlogits + t * E;
  int ids[KMAX];
  float g[KMAX], w[KMAX];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      ids[j] = topk_idx[t * k + j];
      g[j] = dtopk_w[t * k + j];
      w[j] = topk_w[t * k + j];
      s = fmaf(w[j], g[j], s);
    }
  }
  if (renorm) {
    if (!accumulate) {
      if ((E & 3) == 0)
        for (int e = 0; e < E; e += 4) *reinterpret_cast<float4 *>(drow + e) = make_float4(0.f, 0.f, 0.f, 0.f);
      else
        for (int e = 0; e < E; ++e) drow[e] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) drow[ids[j]] = accumulate ? drow[ids[j]] + w[j] * (g[j] - s) : w[j] * (g[j] - s);
    return;
  }
  // accumulate: what dlogits held at the selected ids, before the first pass
  float base[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) base[j] = (accumulate && j < k) ? drow[ids[j]] : 0.f;
  float m = -INFINITY;
  for_row(row, E, [&](int, float l) {
    if (l == l) m = fmaxf(m, l);
  });
  float sum = 0.f;
  for_row(row, E, [&](int, float l) { sum += (l == l) ? expf(l - m) : 0.f; });
  const float inv = 1.f / sum;
  auto dval = [&](float l, float old) {
    const float p = (l == l) ? expf(l - m) * inv : 0.f;
    return accumulate ? old - p * s : -p * s;
  };
  if ((E & 3) == 0) {  // 16-byte rows: four values per load and store
    for (int e = 0; e < E; e += 4) {
      const float4 l = *reinterpret_cast<const float4 *>(row + e);
      float4 o = {0.f, 0.f, 0.f, 0.f};
      if (accumulate) o = *reinterpret_cast<const float4 *>(drow + e);
      *reinterpret_cast<float4 *>(drow + e) =
          make_float4(dval(l.x, o.x), dval(l.y, o.y), dval(l.z, o.z), dval(l.w, o.w));
    }
  } else {
    for (int e = 0; e < E; ++e) drow[e] = dval(row[e], accumulate ? drow[e] : 0.f);
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      float l = row[ids[j]];
      float p = (l == l) ? expf(l - m) * inv : 0.f;
      drow[ids[j]] = accumulate ? base[j] + p * (g[j] - s) : p * (g[j] - s);
    }
  }
}

// Router backward: dx_router[t,c] = sum_e dlogits[t,e] w_router[e,c].
template <typename T>
__global__ __launch_bounds__(256) void router_dx_kernel(const float *__restrict__ dlogits,
                                                        const T *__restrict__ wr, float *__restrict__ dx,
                                                        int64_t ntok, int d, int E) {
  const int c = blockIdx.y * 256 + threadIdx.x;
  const int64_t t = blockIdx.x;
  if (c >= d || t >= ntok) return;
  float acc = 0.f;
  for (int e = 0; e < E; ++e) acc = fmaf(dlogits[t * E + e], Elem<T>::load(wr + (size_t)e * d + c), acc);
  dx[t * d + c] = acc;
}

// Router weight gradient, pass 1: partial[chunk, e, c] = sum over the
// chunk's tokens of dlogits[t,e] x[t,c]; 8 experts per thread.
template <typename T>
__global__ __launch_bounds__(256) void router_dw_partial_kernel(const float *__restrict__ dlogits,
                                                                const T *__restrict__ x,
                                                                float *__restrict__ partial, int64_t ntok,
                                                                int d, int E, int64_t chunk_tokens) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int64_t chunk = blockIdx.y;
  const int e0 = blockIdx.z * 8;
  if (c >= d) return;
  const int64_t t0 = chunk * chunk_tokens;
  const int64_t t1 = t0 + chunk_tokens < ntok ? t0 + chunk_tokens : ntok;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int64_t t = t0; t < t1; ++t) {
    const float xv = Elem<T>::load(x + t * d + c);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (e0 + i < E) acc[i] = fmaf(dlogits[t * E + e0 + i], xv, acc[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (e0 + i < E) partial[(chunk * E + e0 + i) * (int64_t)d + c] = acc[i];
}

// Router weight gradient, pass 2: dw_router[e,c] += sum over chunks, in
// chunk order.
__global__ __launch_bounds__(256) void router_dw_reduce_kernel(const float *__restrict__ partial,
                                                               float *__restrict__ dw, int64_t nchunk, int d,
                                                               int E) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int e = blockIdx.y;
  if (c >= d) return;
  float acc = 0.f;
  for (int64_t ch = 0; ch < nchunk; ++ch) acc += partial[(ch * E + e) * (int64_t)d + c];
  dw[(int64_t)e * d + c] += acc;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_router_logits(const void *x, const void *w_router, const float *bias, float *logits,
                                int64_t T, int d, int E, bool bf16, hipStream_t s) {
  LaunchScope scope("router_logits", s);
  dim3 grid((unsigned)((T + 3) / 4));
  if (bf16)
    router_logits_kernel<bf16_t><<<grid, 256, 0, s>>>((const bf16_t *)x, (const bf16_t *)w_router, bias, logits,
                                                      T, d, E);
  else
    router_logits_kernel<float><<<grid, 256, 0, s>>>((const float *)x, (const float *)w_router, bias, logits, T,
                                                     d, E);
  return hipGetLastError();
}

template <int KMAX>
static void launch_topk_k(const float *logits, int32_t *topk_idx, float *topk_w, int32_t *rank, int32_t *blk_cnt,
                          int64_t T, int E, int k, bool renorm, hipStream_t s) {
  dim3 grid((unsigned)route_blocks(T));
  route_topk_kernel<KMAX><<<grid, kRouteTokensPerBlock, 0, s>>>(logits, topk_idx, topk_w, rank, blk_cnt, T, E, k,
                                                                 renorm ? 1 : 0);
}

// Scratch of the allocation-free routing entry point (moe_route_noalloc):
// the per-workgroup expert histograms, kRouteScratchBytes in device memory
// that every GPU the library runs on holds until the process ends. In host
// code `scratch` names a host-side stand-in, not a device address: the
// kernels only ever get the address hipGetSymbolAddress returns for the
// current device. The route pass writes every histogram entry it reads, so
// nothing has to be cleared between calls.
static __device__ __align__(256) int32_t scratch[kRouteScratchBytes / sizeof(int32_t)];

hipError_t route_scratch(int32_t **out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int32_t *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {  // once per device, with that device current
    void *p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    addr[dev] = static_cast<int32_t *>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_route(const float *logits, int32_t *topk_idx, float *topk_w, int32_t *counts,
                        int32_t *offsets, int32_t *row_of_slot, int32_t *src_of_row, int32_t *blk_cnt,
                        int64_t T, int E, int k, bool renorm, hipStream_t s) {
  const int64_t nblk = route_blocks(T);
  {
    LaunchScope scope("route_topk", s);
    if (k <= 1)
      launch_topk_k<1>(logits, topk_idx, topk_w, row_of_slot, blk_cnt, T, E, k, renorm, s);
    else if (k <= 2)
      launch_topk_k<2>(logits, topk_idx, topk_w, row_of_slot, blk_cnt, T, E, k, renorm, s);
    else if (k <= 4)
      launch_topk_k<4>(logits, topk_idx, topk_w, row_of_slot, blk_cnt, T, E, k, renorm, s);
    else if (k <= 8)
      launch_topk_k<8>(logits, topk_idx, topk_w, row_of_slot, blk_cnt, T, E, k, renorm, s);
    else
      launch_topk_k<16>(logits, topk_idx, topk_w, row_of_slot, blk_cnt, T, E, k, renorm, s);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  {
    LaunchScope scope("route_scan", s);
    route_scan_kernel<<<dim3((unsigned)E), 256, 0, s>>>(blk_cnt, counts, nblk, E);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t nslot = T * k;
  {
    LaunchScope scope("route_rows", s);
    route_rows_kernel<<<dim3((unsigned)((nslot + 255) / 256)), 256, 0, s>>>(topk_idx, counts, blk_cnt, row_of_slot,
                                                                          src_of_row, offsets, nslot, E, k);
  }
  return hipGetLastError();
}

hipError_t launch_route_bwd(const float *dtopk_w, const float *logits, const int32_t *topk_idx,
                            const float *topk_w, float *dlogits, int64_t T, int E, int k, bool renorm,
                            bool accumulate, hipStream_t s) {
  LaunchScope scope("route_bwd", s);
  dim3 grid((unsigned)((T + kRouteBwdThreads - 1) / kRouteBwdThreads));
  const int r = renorm ? 1 : 0, a = accumulate ? 1 : 0;
  if (k <= 2)
    route_bwd_kernel<2><<<grid, kRouteBwdThreads, 0, s>>>(dtopk_w, logits, topk_idx, topk_w, dlogits, T, E, k, r, a);
  else if (k <= 4)
    route_bwd_kernel<4><<<grid, kRouteBwdThreads, 0, s>>>(dtopk_w, logits, topk_idx, topk_w, dlogits, T, E, k, r, a);
  else if (k <= 8)
    route_bwd_kernel<8><<<grid, kRouteBwdThreads, 0, s>>>(dtopk_w, logits, topk_idx, topk_w, dlogits, T, E, k, r, a);
  else
    route_bwd_kernel<16><<<grid, kRouteBwdThreads, 0, s>>>(dtopk_w, logits, topk_idx, topk_w, dlogits, T, E, k, r, a);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const float *dlogits, const void *x, const void *w_router, float *dx_router,
                             float *dw_router, float *partial, int64_t T, int d, int E, bool bf16,
                             hipStream_t s) {
  const int64_t chunk = router_chunk_tokens(T);
  const int64_t nchunk = router_chunks(T);
  const unsigned cblocks = (unsigned)((d + 255) / 256);
  {
    LaunchScope scope("router_dx", s);
    if (bf16)
      router_dx_kernel<bf16_t><<<dim3((unsigned)T, cblocks), 256, 0, s>>>(dlogits, (const bf16_t *)w_router,
                                                                         dx_router, T, d, E);
    else
      router_dx_kernel<float><<<dim3((unsigned)T, cblocks), 256, 0, s>>>(dlogits, (const float *)w_router,
                                                                        dx_router, T, d, E);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  {
    LaunchScope scope("router_dw_partial", s);
    dim3 grid(cblocks, (unsigned)nchunk, (unsigned)((E + 7) / 8));
    if (bf16)
      router_dw_partial_kernel<bf16_t><<<grid, 256, 0, s>>>(dlogits, (const bf16_t *)x, partial, T, d, E, chunk);
    else
      router_dw_partial_kernel<float><<<grid, 256, 0, s>>>(dlogits, (const float *)x, partial, T, d, E, chunk);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  {
    LaunchScope scope("router_dw_reduce", s);
    router_dw_reduce_kernel<<<dim3(cblocks, (unsigned)E), 256, 0, s>>>(partial, dw_router, nchunk, d, E);
  }
  return hipGetLastError();
}

}  // namespace moe
