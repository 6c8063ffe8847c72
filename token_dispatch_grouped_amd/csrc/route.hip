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
#include "route_lane.h"

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

// Inverse of order_key: the logit a key stands for (-0.0 comes back as +0.0,
// every NaN as one NaN).
MOE_DEVICE float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

MOE_DEVICE uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
MOE_DEVICE uint64_t min_u64(uint64_t a, uint64_t b) { return a > b ? b : a; }

// Bitonic sorting network over N (a power of two) keys, descending.
template <int N>
MOE_DEVICE void sort_desc(uint64_t (&c)[N]) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
    for (int stride = size / 2; stride > 0; stride >>= 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const uint64_t x = c[i], y = c[j];
          const bool desc = (i & size) == 0;  // the last stage sorts all N descending
          c[i] = desc ? max_u64(x, y) : min_u64(x, y);
          c[j] = desc ? min_u64(x, y) : max_u64(x, y);
        }
      }
    }
  }
}

// Keep the KMAX largest of two descending key lists in `a`, descending. The
// larger of a[i] and b[KMAX-1-i] over all i are the KMAX largest of both
// lists and form a bitonic sequence, which log2(KMAX) half-cleaner stages put
// in descending order. Swapping the two lists gives the same result.
template <int KMAX>
MOE_DEVICE void merge_topk(uint64_t (&a)[KMAX], const uint64_t (&b)[KMAX]) {
#pragma unroll
  for (int i = 0; i < KMAX; ++i) a[i] = max_u64(a[i], b[KMAX - 1 - i]);
#pragma unroll
  for (int h = KMAX / 2; h > 0; h >>= 1) {
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if ((i & h) == 0) {
        const uint64_t x = a[i], y = a[i + h];
        a[i] = max_u64(x, y);
        a[i + h] = min_u64(x, y);
      }
    }
  }
}

// merge_topk with the list of the lane `s` away (same wavefront).
template <int KMAX>
MOE_DEVICE void merge_topk_xor(uint64_t (&a)[KMAX], int s) {
  uint64_t b[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    const uint32_t lo = __shfl_xor((uint32_t)a[i], s);
    const uint32_t hi = __shfl_xor((uint32_t)(a[i] >> 32), s);
    b[i] = ((uint64_t)hi << 32) | lo;
  }
  merge_topk<KMAX>(a, b);
}

// The KMAX largest of V keys (V a multiple of 8), descending, padded with 0:
// each run of eight sorted by a network, the runs' KMAX largest merged.
template <int KMAX, int V>
MOE_DEVICE void local_topk(const uint64_t (&c)[V], uint64_t (&list)[KMAX]) {
#pragma unroll
  for (int r = 0; r < V / 8; ++r) {
    uint64_t run[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) run[i] = c[8 * r + i];
    sort_desc<8>(run);
    uint64_t top[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) top[i] = i < 8 ? run[i] : 0ull;
    if (r == 0) {
#pragma unroll
      for (int i = 0; i < KMAX; ++i) list[i] = top[i];
    } else {
      merge_topk<KMAX>(list, top);
    }
  }
}

// ---------------------------------------------------------------------------
// A2 + first half of A3: per token top-k and weights; per workgroup the
// stable rank of each (token, slot) among the workgroup's slots of the same
// expert, and the workgroup's expert histogram.
//
// kRouteTokensPerBlock tokens per workgroup, G = route_lanes(E) lanes per
// token. A lane reads its share of the logit row in one round of 16-byte
// loads and sorts the 64-bit composite keys of its share (logit key, then
// inverted id, so that the lower id wins a tie) in runs of eight with a
// sorting network, keeping the k largest; the G lanes then merge their k
// largest pairwise over a butterfly, after which every lane holds the token's
// top k. The softmax maximum is the first key's logit; the
// sum of exponentials is added up per lane and then over the butterfly (each
// pair adds the same two terms, so every lane gets the same sum). Lane g
// writes slots g, g + G, ...
//
// A token selects an expert at most once, so the rank of slot (t, j) among
// the workgroup's slots of expert e is the number of earlier tokens of the
// workgroup that selected e: each slot sets its token's bit in expert e's
// 64-bit mask in LDS (bitwise OR, whose result does not depend on the order
// of the updates) and the rank is the population count of the mask below the
// token's bit. No atomic decides any order.
// ---------------------------------------------------------------------------
template <int KMAX, int G, int V>
__global__ __launch_bounds__(kRouteTokensPerBlock *G) void route_topk_kernel(const float *__restrict__ logits,
                                                                 int32_t *__restrict__ topk_idx,
                                                                 float *__restrict__ topk_w,
                                                                 int32_t *__restrict__ local_rank,
                                                                 int32_t *__restrict__ blk_cnt, int64_t ntok,
                                                                 int E, int k, int renorm) {
  static_assert(kRouteTokensPerBlock == 64, "one bit per token of the workgroup in a 64-bit mask");
  constexpr int NT = kRouteTokensPerBlock * G;
  using Lane = RouteLane<G, V>;
  __shared__ unsigned long long s_mask[256];
  const int tid = threadIdx.x;
  const int g = tid % G;
  const int tl = tid / G;  // token within the workgroup
  const int64_t t = (int64_t)blockIdx.x * kRouteTokensPerBlock + tl;
  const bool valid = t < ntok;  // the same for the G lanes of a token
  const bool vec = (E & 3) == 0;

  for (int i = tid; i < E; i += NT) s_mask[i] = 0ull;

  float v[V];
  uint64_t c[V];
  if (valid) Lane::load(logits + t * E, E, g, vec, v);
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = Lane::elem(i, g, vec);
    // 0 lies below every real key: values past the row and rows past the end
    c[i] = (valid && e < E) ? ((uint64_t)order_key(v[i]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e) : 0ull;
  }
  uint64_t list[KMAX];
  local_topk<KMAX, V>(c, list);
#pragma unroll
  for (int s = 1; s < G; s <<= 1) merge_topk_xor<KMAX>(list, s);

  int ids[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) ids[i] = (int)(0xffffffffu - (uint32_t)(list[i] & 0xffffffffu));
  if (valid) {
    // softmax over the whole row; the first selected logit is the maximum
    const float m = key_value((uint32_t)(list[0] >> 32));
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = Lane::elem(i, g, vec);
      if (e < E && v[i] == v[i]) sum += expf(v[i] - m);
    }
#pragma unroll
    for (int s = 1; s < G; s <<= 1) sum += __shfl_xor(sum, s);
    float w[KMAX];
    float wsum = 0.f;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      const float l = key_value((uint32_t)(list[i] >> 32));
      w[i] = (i < k && l == l) ? expf(l - m) / sum : 0.f;
      if (i < k) wsum += w[i];
    }
    if (renorm) {
#pragma unroll
      for (int i = 0; i < KMAX; ++i) w[i] = w[i] / wsum;
    }
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (i < k && i % G == g) {
        topk_idx[t * k + i] = ids[i];
        topk_w[t * k + i] = w[i];
      }
    }
  }
  __syncthreads();  // masks cleared
  if (valid) {
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (i < k && i % G == g) atomicOr(&s_mask[ids[i]], 1ull << tl);
  }
  __syncthreads();
  if (valid) {
    const uint64_t below = (1ull << tl) - 1ull;
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (i < k && i % G == g) local_rank[t * k + i] = __popcll(s_mask[ids[i]] & below);
  }
  for (int e = tid; e < E; e += NT) blk_cnt[(int64_t)blockIdx.x * E + e] = __popcll(s_mask[e]);
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
// B2: dlogits from dtopk_w. route_lanes(E) lanes per token as in the top-k:
// each lane holds its share of the logit row in registers, the row maximum
// and the sum of exponentials are reduced over the token's lanes, and each
// lane writes its share of the dlogits row.
// ---------------------------------------------------------------------------
constexpr int kRouteBwdThreads = 256;

template <int KMAX, int G, int V>
__global__ __launch_bounds__(kRouteBwdThreads) void route_bwd_kernel(const float *__restrict__ dtopk_w,
                                                        const float *__restrict__ logits,
                                                        const int32_t *__restrict__ topk_idx,
                                                        const float *__restrict__ topk_w,
                                                        float *__restrict__ dlogits, int64_t ntok, int E, int k,
                                                        int renorm, int accumulate) {
  using Lane = RouteLane<G, V>;
  const int g = threadIdx.x % G;
  const int64_t t = ((int64_t)blockIdx.x * kRouteBwdThreads + threadIdx.x) / G;
  // a token's G lanes leave together, so the reductions below only ever
  // exchange values between lanes that stay
  if (t >= ntok) return;
  const bool vec = (E & 3) == 0;
  const float *row = logits + t * E;
  float *drow = dlogits + t * E;
  int ids[KMAX];
  float gk[KMAX], wk[KMAX];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    ids[j] = -1;
    gk[j] = wk[j] = 0.f;
    if (j < k) {
      ids[j] = topk_idx[t * k + j];
      gk[j] = dtopk_w[t * k + j];
      wk[j] = topk_w[t * k + j];
      s = fmaf(wk[j], gk[j], s);
    }
  }
  float old[V];
  if (accumulate)
    Lane::load(drow, E, g, vec, old);
  else
#pragma unroll
    for (int i = 0; i < V; ++i) old[i] = 0.f;
  float d[V];
  if (renorm) {
    // only the selected logits carry a gradient: w_j (g_j - s)
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = Lane::elem(i, g, vec);
      bool sel = false;
      float x = 0.f;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (ids[j] == e) {
          sel = true;
          x = wk[j] * (gk[j] - s);
        }
      }
      d[i] = sel ? (accumulate ? old[i] + x : x) : old[i];
    }
  } else {
    float l[V];
    Lane::load(row, E, g, vec, l);
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (Lane::elem(i, g, vec) < E && l[i] == l[i]) m = fmaxf(m, l[i]);
#pragma unroll
    for (int o = 1; o < G; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (Lane::elem(i, g, vec) < E && l[i] == l[i]) sum += expf(l[i] - m);
#pragma unroll
    for (int o = 1; o < G; o <<= 1) sum += __shfl_xor(sum, o);
    const float inv = 1.f / sum;
    // p_e (g_e - s): g_e = dtopk_w of the slot that selected e, else 0
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = Lane::elem(i, g, vec);
      const float p = (l[i] == l[i]) ? expf(l[i] - m) * inv : 0.f;
      bool sel = false;
      float ge = 0.f;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (ids[j] == e) {
          sel = true;
          ge = gk[j];
        }
      }
      const float x = sel ? p * (ge - s) : -(p * s);
      d[i] = accumulate ? old[i] + x : x;
    }
  }
  if (vec) {
#pragma unroll
    for (int c = 0; c < V / 4; ++c) {
      const int e = 4 * (g + G * c);
      if (e < E)
        *reinterpret_cast<float4 *>(drow + e) = make_float4(d[4 * c], d[4 * c + 1], d[4 * c + 2], d[4 * c + 3]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = g + G * i;
      if (e < E) drow[e] = d[i];
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

template <int KMAX, int G, int V>
static void launch_topk_kg(const float *logits, int32_t *topk_idx, float *topk_w, int32_t *rank, int32_t *blk_cnt,
                           int64_t T, int E, int k, int r, hipStream_t s) {
  route_topk_kernel<KMAX, G, V><<<dim3((unsigned)route_blocks(T)), kRouteTokensPerBlock * G, 0, s>>>(
      logits, topk_idx, topk_w, rank, blk_cnt, T, E, k, r);
}

template <int KMAX>
static void launch_topk_k(const float *logits, int32_t *topk_idx, float *topk_w, int32_t *rank, int32_t *blk_cnt,
                          int64_t T, int E, int k, bool renorm, hipStream_t s) {
  const int r = renorm ? 1 : 0;
  switch (route_lanes(E) * route_lane_values(E)) {  // (G, V): (1, 8) (2, 8) (4, 8) (8, 8) (8, 16) (8, 32)
    case 8: launch_topk_kg<KMAX, 1, 8>(logits, topk_idx, topk_w, rank, blk_cnt, T, E, k, r, s); break;
    case 16: launch_topk_kg<KMAX, 2, 8>(logits, topk_idx, topk_w, rank, blk_cnt, T, E, k, r, s); break;
    case 32: launch_topk_kg<KMAX, 4, 8>(logits, topk_idx, topk_w, rank, blk_cnt, T, E, k, r, s); break;
    case 64: launch_topk_kg<KMAX, 8, 8>(logits, topk_idx, topk_w, rank, blk_cnt, T, E, k, r, s); break;
    case 128: launch_topk_kg<KMAX, 8, 16>(logits, topk_idx, topk_w, rank, blk_cnt, T, E, k, r, s); break;
    default: launch_topk_kg<KMAX, 8, 32>(logits, topk_idx, topk_w, rank, blk_cnt, T, E, k, r, s); break;
  }
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

template <int KMAX, int G, int V>
static void launch_route_bwd_kg(const float *dtopk_w, const float *logits, const int32_t *topk_idx,
                                const float *topk_w, float *dlogits, int64_t T, int E, int k, int r, int a,
                                hipStream_t s) {
  const dim3 grid((unsigned)((T * G + kRouteBwdThreads - 1) / kRouteBwdThreads));
  route_bwd_kernel<KMAX, G, V><<<grid, kRouteBwdThreads, 0, s>>>(dtopk_w, logits, topk_idx, topk_w, dlogits, T, E, k,
                                                              r, a);
}

template <int KMAX>
static void launch_route_bwd_k(const float *dtopk_w, const float *logits, const int32_t *topk_idx,
                               const float *topk_w, float *dlogits, int64_t T, int E, int k, int r, int a,
                               hipStream_t s) {
  switch (route_lanes(E) * route_lane_values(E)) {  // (G, V) as in the top-k
    case 8: launch_route_bwd_kg<KMAX, 1, 8>(dtopk_w, logits, topk_idx, topk_w, dlogits, T, E, k, r, a, s); break;
    case 16: launch_route_bwd_kg<KMAX, 2, 8>(dtopk_w, logits, topk_idx, topk_w, dlogits, T, E, k, r, a, s); break;
    case 32: launch_route_bwd_kg<KMAX, 4, 8>(dtopk_w, logits, topk_idx, topk_w, dlogits, T, E, k, r, a, s); break;
    case 64: launch_route_bwd_kg<KMAX, 8, 8>(dtopk_w, logits, topk_idx, topk_w, dlogits, T, E, k, r, a, s); break;
    case 128: launch_route_bwd_kg<KMAX, 8, 16>(dtopk_w, logits, topk_idx, topk_w, dlogits, T, E, k, r, a, s); break;
    default: launch_route_bwd_kg<KMAX, 8, 32>(dtopk_w, logits, topk_idx, topk_w, dlogits, T, E, k, r, a, s); break;
  }
}

hipError_t launch_route_bwd(const float *dtopk_w, const float *logits, const int32_t *topk_idx,
                            const float *topk_w, float *dlogits, int64_t T, int E, int k, bool renorm,
                            bool accumulate, hipStream_t s) {
  LaunchScope scope("route_bwd", s);
  const int r = renorm ? 1 : 0, a = accumulate ? 1 : 0;
  if (k <= 2)
    launch_route_bwd_k<2>(dtopk_w, logits, topk_idx, topk_w, dlogits, T, E, k, r, a, s);
  else if (k <= 4)
    launch_route_bwd_k<4>(dtopk_w, logits, topk_idx, topk_w, dlogits, T, E, k, r, a, s);
  else if (k <= 8)
    launch_route_bwd_k<8>(dtopk_w, logits, topk_idx, topk_w, dlogits, T, E, k, r, a, s);
  else
    launch_route_bwd_k<16>(dtopk_w, logits, topk_idx, topk_w, dlogits, T, E, k, r, a, s);
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
