// MoE auxiliary losses and routing metrics (latency-bound, two launches).
//
// Pass 1 (aux_partial_kernel): each token's row is shared by route_lanes(E)
// lanes (the routing kernels' split: at most 8 values per lane for E <= 64).
// Per token it forms the full softmax p and lse = log sum exp(logits), the
// row maximum and the sums reduced over the token's lanes, adds p into
// per-lane sums of P_e, lse^2, the entropy -sum p log p (log p taken as
// logit - lse) and the top probability (= exp(max - lse)), and, if asked,
// writes the gradient
//   dlogits[t,i] = p_i (G_i - sum_e p_e G_e) + (2 beta / T) lse p_i,
//   G_e = alpha E counts[e] / (T^2 k)     (d(alpha L_bal)/dp[t,e])
// overwriting or adding to dlogits. Each workgroup covers a contiguous run
// of tokens; its sums are combined over token groups and wavefronts in a
// fixed order into one partial row [E + 3] per workgroup.
// Pass 2 (aux_finalize_kernel, one workgroup): partial rows summed in eight
// interleaved chains combined in a fixed order, count statistics, losses and
// the metrics array.
// No atomics: results are the same run to run.
#include <math.h>

#include "common.h"
#include "kernels.h"
#include "route_lane.h"

namespace moe {

constexpr int kAuxThreads = 256;
constexpr int kAuxMaxE = 256;
constexpr int kAuxScalars = 3;                 // entropy, lse^2, top probability

// Sum / maximum over the G lanes of one token (aligned groups of G lanes).
template <int G>
MOE_DEVICE float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < G; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
template <int G>
MOE_DEVICE float group_max(float v) {
#pragma unroll
  for (int o = 1; o < G; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

template <int G, int V>
__global__ __launch_bounds__(kAuxThreads) void aux_partial_kernel(const float *__restrict__ logits,
                                                                  const int32_t *__restrict__ counts,
                                                                  float *__restrict__ partial, float *dlogits,
                                                                  int64_t T, int E, int tokens_per_block,
                                                                  float gscale, float zscale, int accumulate) {
  using Lane = RouteLane<G, V>;
  constexpr int TPI = kAuxThreads / G;  // tokens of the workgroup per iteration
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int g = threadIdx.x % G;
  const bool vec = (E & 3) == 0;
  const int64_t t0 = (int64_t)blockIdx.x * tokens_per_block;
  int64_t t_end = t0 + tokens_per_block;
  if (t_end > T) t_end = T;
  float Gv[V], psum[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = Lane::elem(i, g, vec);
    Gv[i] = (dlogits && e < E) ? gscale * (float)counts[e] : 0.f;
    psum[i] = 0.f;
  }
  float ent = 0.f, zz = 0.f, mx = 0.f;
  // a token's G lanes take the same tokens, so the reductions below stay
  // within lanes that are all active
  for (int64_t t = t0 + threadIdx.x / G; t < t_end; t += TPI) {
    const float *row = logits + t * E;
    float l[V], old[V];
    Lane::load(row, E, g, vec, l);
    if (dlogits && accumulate) Lane::load(dlogits + t * E, E, g, vec, old);
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      if (Lane::elem(i, g, vec) >= E) l[i] = -INFINITY;  // past the row: exp gives 0
      m = fmaxf(m, l[i]);
    }
    m = group_max<G>(m);
    float ex[V], sm = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      ex[i] = expf(l[i] - m);
      sm += ex[i];
    }
    sm = group_sum<G>(sm);
    const float inv = 1.f / sm;
    const float lse = m + logf(sm);
    float p[V], plogp = 0.f, pg = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      p[i] = ex[i] * inv;
      if (p[i] > 0.f) plogp += p[i] * (l[i] - lse);
      pg += p[i] * Gv[i];
      psum[i] += p[i];
    }
    plogp = group_sum<G>(plogp);
    if (dlogits) {
      pg = group_sum<G>(pg);
      float d[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const float v = p[i] * (Gv[i] - pg) + zscale * lse * p[i];
        d[i] = accumulate ? old[i] + v : v;
      }
      float *drow = dlogits + t * E;
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
    if (g == 0) {  // the token's scalars once
      ent -= plogp;
      zz += lse * lse;
      mx += inv;  // the top probability is exp(m - lse) = 1 / s
    }
  }
  // P_e: lanes g of every token group hold the same experts; add over the
  // wavefront's token groups, then over the wavefronts, in a fixed order
#pragma unroll
  for (int i = 0; i < V; ++i)
#pragma unroll
    for (int o = G; o < kWave; o <<= 1) psum[i] += __shfl_xor(psum[i], o, kWave);
  ent = wave_sum(ent);
  zz = wave_sum(zz);
  mx = wave_sum(mx);
  __shared__ float sp[kAuxThreads / kWave][kAuxMaxE];
  __shared__ float ss[kAuxThreads / kWave][kAuxScalars];
  if (lane < G) {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = Lane::elem(i, g, vec);
      if (e < E) sp[wv][e] = psum[i];
    }
  }
  if (lane == 0) {
    ss[wv][0] = ent;
    ss[wv][1] = zz;
    ss[wv][2] = mx;
  }
  __syncthreads();
  float *out = partial + (int64_t)blockIdx.x * (E + kAuxScalars);
  for (int e = threadIdx.x; e < E; e += kAuxThreads) out[e] = ((sp[0][e] + sp[1][e]) + sp[2][e]) + sp[3][e];
  if (threadIdx.x < kAuxScalars) {
    const int i = threadIdx.x;
    out[E + i] = ((ss[0][i] + ss[1][i]) + ss[2][i]) + ss[3][i];
  }
}

// Fixed-order tree sum over the 256 threads of the workgroup.
MOE_DEVICE float block_sum_256(float v, float *red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int o = kAuxThreads / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

MOE_DEVICE float block_max_256(float v, float *red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int o = kAuxThreads / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kAuxThreads) void aux_finalize_kernel(const float *__restrict__ partial, int nblk,
                                                                   const int32_t *__restrict__ counts, int64_t T,
                                                                   int E, int k, float *losses, float *metrics) {
  __shared__ float red[kAuxThreads];
  // column sums of the partial rows: eight interleaved chains per column
  // (rows r mod 8, ascending), combined in a fixed order; thread t takes
  // chain t / 32 of column t % 32 of each pass over 32 columns, so that a
  // row's columns are read together
  constexpr int kChains = 8;
  constexpr int kCols = kAuxThreads / kChains;
  __shared__ float chain[kChains][kAuxMaxE + kAuxScalars];
  const int ld = E + kAuxScalars;
  for (int c0 = 0; c0 < ld; c0 += kCols) {
    const int col = c0 + (int)threadIdx.x % kCols;
    const int r = (int)threadIdx.x / kCols;
    if (col < ld) {
      float acc = 0.f;
#pragma unroll 8
      for (int b = r; b < nblk; b += kChains) acc += partial[(int64_t)b * ld + col];
      chain[r][col] = acc;
    }
  }
  __syncthreads();
  auto column = [&](int col) {
    return ((chain[0][col] + chain[1][col]) + (chain[2][col] + chain[3][col])) +
           ((chain[4][col] + chain[5][col]) + (chain[6][col] + chain[7][col]));
  };
  const int e = threadIdx.x;  // E <= 256: one expert per thread
  const float Tf = (float)T;
  const float rows = (float)((double)T * k);
  const float mean = (float)((double)T * k / E);
  float fP = 0.f, dev2 = 0.f, cmax = 0.f, empty = 0.f;
  if (e < E) {
    const float P = column(e) / Tf;
    const float c = (float)counts[e];
    const float f = c / rows;
    fP = f * P;
    dev2 = (c - mean) * (c - mean);
    cmax = c;
    empty = counts[e] == 0 ? 1.f : 0.f;
    if (metrics) {
      metrics[MOE_METRIC_SCALARS + e] = f;
      metrics[MOE_METRIC_SCALARS + E + e] = P;
    }
  }
  const float sc = e < kAuxScalars ? column(E + e) : 0.f;
  const float sum_fP = block_sum_256(fP, red);
  const float sum_dev2 = block_sum_256(dev2, red);
  const float sum_empty = block_sum_256(empty, red);
  const float max_c = block_max_256(cmax, red);
  // scalars from threads 0..2 -> shared
  __shared__ float scal[kAuxScalars];
  if (e < kAuxScalars) scal[e] = sc / Tf;
  __syncthreads();
  if (e == 0) {
    if (losses) {
      losses[0] = (float)E * sum_fP;
      losses[1] = scal[1];
    }
    if (metrics) {
      metrics[MOE_METRIC_IMBALANCE] = max_c / mean;
      metrics[MOE_METRIC_EMPTY_EXPERTS] = sum_empty;
      metrics[MOE_METRIC_COUNT_CV] = sqrtf(sum_dev2 / (float)E) / mean;
      metrics[MOE_METRIC_ENTROPY] = scal[0];
      metrics[MOE_METRIC_MAX_PROB] = scal[2];
    }
  }
}

// An empty microbatch: both losses 0, every metric 0 except the number of
// empty experts, which is E (no expert has a row).
__global__ __launch_bounds__(kAuxThreads) void aux_empty_kernel(float *losses, float *metrics, int E) {
  const int i = threadIdx.x;
  if (losses && i < 2) losses[i] = 0.f;
  if (metrics)
    for (int q = i; q < MOE_METRIC_SCALARS + 2 * E; q += kAuxThreads)
      metrics[q] = q == MOE_METRIC_EMPTY_EXPERTS ? (float)E : 0.f;
}

template <int G, int V>
static void aux_partial_t(const float *logits, const int32_t *counts, float *partial, float *dlogits, int64_t T,
                          int E, int tpb, int nblk, float gscale, float zscale, int acc, hipStream_t s) {
  aux_partial_kernel<G, V><<<nblk, kAuxThreads, 0, s>>>(logits, counts, partial, dlogits, T, E, tpb, gscale, zscale,
                                                        acc);
}

hipError_t launch_aux_loss(const float *logits, const int32_t *counts, float *losses, float *metrics, float *dlogits,
                           float *partial, int64_t T, int E, int k, float alpha, float beta, bool accumulate,
                           hipStream_t s) {
  if (T == 0) {  // no rows of dlogits; the losses and metrics of no tokens
    if (!losses && !metrics) return hipSuccess;
    LaunchScope scope("aux_empty", s);
    aux_empty_kernel<<<1, kAuxThreads, 0, s>>>(losses, metrics, E);
    return hipGetLastError();
  }
  const int tpb = aux_tokens_per_block(T);
  const int nblk = (int)((T + tpb - 1) / tpb);
  const float gscale = (float)((double)alpha * E / ((double)T * (double)T * k));
  const float zscale = (float)(2.0 * beta / (double)T);
  {
    LaunchScope scope("aux_partial", s);
    const int acc = accumulate ? 1 : 0;
    switch (route_lanes(E) * route_lane_values(E)) {  // (G, V): (1, 8) (2, 8) (4, 8) (8, 8) (8, 16) (8, 32)
      case 8: aux_partial_t<1, 8>(logits, counts, partial, dlogits, T, E, tpb, nblk, gscale, zscale, acc, s); break;
      case 16: aux_partial_t<2, 8>(logits, counts, partial, dlogits, T, E, tpb, nblk, gscale, zscale, acc, s); break;
      case 32: aux_partial_t<4, 8>(logits, counts, partial, dlogits, T, E, tpb, nblk, gscale, zscale, acc, s); break;
      case 64: aux_partial_t<8, 8>(logits, counts, partial, dlogits, T, E, tpb, nblk, gscale, zscale, acc, s); break;
      case 128: aux_partial_t<8, 16>(logits, counts, partial, dlogits, T, E, tpb, nblk, gscale, zscale, acc, s); break;
      default: aux_partial_t<8, 32>(logits, counts, partial, dlogits, T, E, tpb, nblk, gscale, zscale, acc, s); break;
    }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || (!losses && !metrics)) return err;
  {
    LaunchScope scope("aux_finalize", s);
    aux_finalize_kernel<<<1, kAuxThreads, 0, s>>>(partial, nblk, counts, T, E, k, losses, metrics);
  }
  return hipGetLastError();
}

}  // namespace moe
