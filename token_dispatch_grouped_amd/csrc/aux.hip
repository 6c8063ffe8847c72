// MoE auxiliary losses and routing metrics (latency-bound, two launches).
//
// Pass 1 (aux_partial_kernel): one wavefront per token, lanes across experts
// (lane l holds experts l, l+64, l+128, l+192). Per token it forms the full
// softmax p and lse = log sum exp(logits), adds p into per-lane sums of
// P_e, lse^2, the entropy -sum p log p (log p taken as logit - lse) and the
// top probability (= exp(max - lse)), and, if asked, writes the gradient
//   dlogits[t,i] = p_i (G_i - sum_e p_e G_e) + (2 beta / T) lse p_i,
//   G_e = alpha E counts[e] / (T^2 k)     (d(alpha L_bal)/dp[t,e])
// overwriting or adding to dlogits. Each workgroup covers a contiguous run
// of tokens, its four wavefronts taking every fourth token (four of their
// tokens in flight at a time); their sums are combined in a fixed order into
// one partial row [E + 3] per workgroup.
// Pass 2 (aux_finalize_kernel, one workgroup): partial rows summed in eight
// interleaved chains combined in a fixed order, count statistics, losses and
// the metrics array.
// No atomics: results are the same run to run.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kAuxThreads = 256;
constexpr int kAuxMaxE = 256;
constexpr int kAuxPerLane = kAuxMaxE / kWave;  // experts per lane
constexpr int kAuxScalars = 3;                 // entropy, lse^2, top probability

MOE_DEVICE float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__global__ __launch_bounds__(kAuxThreads) void aux_partial_kernel(const float *__restrict__ logits,
                                                                  const int32_t *__restrict__ counts,
                                                                  float *__restrict__ partial, float *dlogits,
                                                                  int64_t T, int E, int tokens_per_block,
                                                                  float gscale, float zscale, int accumulate) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * tokens_per_block;
  int64_t t_end = t0 + tokens_per_block;
  if (t_end > T) t_end = T;
  float G[kAuxPerLane], psum[kAuxPerLane];
#pragma unroll
  for (int q = 0; q < kAuxPerLane; ++q) {
    const int e = lane + kWave * q;
    G[q] = (dlogits && e < E) ? gscale * (float)counts[e] : 0.f;
    psum[q] = 0.f;
  }
  float ent = 0.f, zz = 0.f, mx = 0.f;
  // The wavefront's tokens t0 + wv + 4 i are taken TB at a time: loads and
  // reductions of the TB tokens are independent chains that overlap; the
  // per-lane sums still take the tokens in order.
  constexpr int TB = 4;
  constexpr int WSTEP = kAuxThreads / kWave;
  for (int64_t tb = t0 + wv; tb < t_end; tb += TB * WSTEP) {
    float l[TB][kAuxPerLane], m[TB];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int64_t t = tb + u * WSTEP;
      m[u] = -INFINITY;
#pragma unroll
      for (int q = 0; q < kAuxPerLane; ++q) {
        const int e = lane + kWave * q;
        l[u][q] = (t < t_end && e < E) ? logits[t * E + e] : -INFINITY;
        m[u] = fmaxf(m[u], l[u][q]);
      }
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) m[u] = wave_max(m[u]);
    float ex[TB][kAuxPerLane], sm[TB];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      sm[u] = 0.f;
#pragma unroll
      for (int q = 0; q < kAuxPerLane; ++q) {
        ex[u][q] = expf(l[u][q] - m[u]);  // 0 for -inf and for lanes past E
        sm[u] += ex[u][q];
      }
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) sm[u] = wave_sum(sm[u]);
    float p[TB][kAuxPerLane], plogp[TB], pg[TB], lse[TB], inv[TB], old[TB][kAuxPerLane];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int64_t t = tb + u * WSTEP;
      inv[u] = 1.f / sm[u];
      lse[u] = m[u] + logf(sm[u]);
      plogp[u] = 0.f;
      pg[u] = 0.f;
#pragma unroll
      for (int q = 0; q < kAuxPerLane; ++q) {
        const int e = lane + kWave * q;
        p[u][q] = ex[u][q] * inv[u];
        if (p[u][q] > 0.f) plogp[u] += p[u][q] * (l[u][q] - lse[u]);
        pg[u] += p[u][q] * G[q];
        old[u][q] = (dlogits && accumulate && t < t_end && e < E) ? dlogits[t * E + e] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      plogp[u] = wave_sum(plogp[u]);
      if (dlogits) pg[u] = wave_sum(pg[u]);
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int64_t t = tb + u * WSTEP;
      if (t >= t_end) break;  // uniform: the rest of the batch is past the run
#pragma unroll
      for (int q = 0; q < kAuxPerLane; ++q) psum[q] += p[u][q];
      ent -= plogp[u];
      zz += lse[u] * lse[u];
      mx += inv[u];  // the top probability is exp(m - lse) = 1 / s
      if (dlogits) {
        float *drow = dlogits + t * E;
#pragma unroll
        for (int q = 0; q < kAuxPerLane; ++q) {
          const int e = lane + kWave * q;
          if (e < E) {
            const float v = p[u][q] * (G[q] - pg[u]) + zscale * lse[u] * p[u][q];
            drow[e] = accumulate ? old[u][q] + v : v;
          }
        }
      }
    }
  }
  __shared__ float sp[kAuxThreads / kWave][kAuxMaxE];
  __shared__ float ss[kAuxThreads / kWave][kAuxScalars];
#pragma unroll
  for (int q = 0; q < kAuxPerLane; ++q) {
    const int e = lane + kWave * q;
    if (e < E) sp[wv][e] = psum[q];
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
  const int e = threadIdx.x;  // E <= 256: one expert per thread
  const int ld = E + kAuxScalars;
  const float Tf = (float)T;
  const float rows = (float)((double)T * k);
  const float mean = (float)((double)T * k / E);
  float fP = 0.f, dev2 = 0.f, cmax = 0.f, empty = 0.f;
  if (e < E) {
    // eight interleaved partial sums (rows b = r mod 8), added in a fixed order
    float P8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int b = 0;
    for (; b + 8 <= nblk; b += 8)
#pragma unroll
      for (int r = 0; r < 8; ++r) P8[r] += partial[(int64_t)(b + r) * ld + e];
    for (int r = 0; b + r < nblk; ++r) P8[r] += partial[(int64_t)(b + r) * ld + e];
    float P = ((P8[0] + P8[1]) + (P8[2] + P8[3])) + ((P8[4] + P8[5]) + (P8[6] + P8[7]));
    P /= Tf;
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
  float sc = 0.f;
  if (e < kAuxScalars) {
    float S8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int b = 0;
    for (; b + 8 <= nblk; b += 8)
#pragma unroll
      for (int r = 0; r < 8; ++r) S8[r] += partial[(int64_t)(b + r) * ld + E + e];
    for (int r = 0; b + r < nblk; ++r) S8[r] += partial[(int64_t)(b + r) * ld + E + e];
    sc = ((S8[0] + S8[1]) + (S8[2] + S8[3])) + ((S8[4] + S8[5]) + (S8[6] + S8[7]));
  }
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
    aux_partial_kernel<<<nblk, kAuxThreads, 0, s>>>(logits, counts, partial, dlogits, T, E, tpb, gscale, zscale,
                                                     accumulate ? 1 : 0);
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
