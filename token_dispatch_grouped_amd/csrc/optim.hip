// Fused AdamW update of fp32 master weights (HBM-bound elementwise pass).
//
// One pass per element reads theta, grad, m, v and writes theta, m, v, the
// bf16 working copy of theta (optional) and a zeroed grad (optional):
// 28 bytes, + 2 with the bf16 copy, + 4 with the zeroing. Adam with
// decoupled weight decay, as PyTorch's AdamW computes it:
//   g = s*grad;  m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*g*g
//   theta = theta*(1 - lr*wd) - (lr/bc1) * m / (sqrt(v)/sqrt(bc2) + eps)
// with bc1 = 1 - b1^t and bc2 = 1 - b2^t computed on the host in double.
// Each thread takes kVecPerThread runs of 4 consecutive elements, all loads
// issued before any arithmetic; consecutive threads take consecutive runs.
// Every access is non-temporal: nothing here is read again by this pass, and
// the streams then stay out of the caches (about 6% faster than cached
// accesses; eight runs per thread, or non-temporal loads alone, are slower).
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kAdamThreads = 256;
constexpr int kVecPerThread = 4;

struct AdamwParams {
  float *theta;
  float *grad;
  float *m;
  float *v;
  bf16_t *lowp;        // NULL: no bf16 copy
  int64_t nvec;        // full runs of 4 elements
  float b1, b2, one_minus_b1, one_minus_b2;
  float decay;         // 1 - lr*wd
  float step_size;     // lr / bc1
  float bc2_sqrt;      // sqrt(bc2)
  float eps;
  float scale;         // gradient multiplier
  int zero_grad;
};

MOE_DEVICE void adamw_elem(const AdamwParams &p, float &th, float g, float &m, float &v) {
  g *= p.scale;
  m = p.b1 * m + p.one_minus_b1 * g;
  v = p.b2 * v + p.one_minus_b2 * (g * g);
  const float denom = sqrtf(v) / p.bc2_sqrt + p.eps;
  th = th * p.decay;
  th = th - p.step_size * (m / denom);
}

__global__ __launch_bounds__(kAdamThreads) void adamw_kernel(AdamwParams p) {
  int64_t idx[kVecPerThread];
  f32x4_t th[kVecPerThread], g[kVecPerThread], m[kVecPerThread], v[kVecPerThread];
  const int64_t base = (int64_t)blockIdx.x * kAdamThreads * kVecPerThread + threadIdx.x;
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    idx[i] = base + (int64_t)i * kAdamThreads;
    const int64_t j = idx[i] < p.nvec ? idx[i] : p.nvec - 1;  // clamped: loads never wait on a branch
    th[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p.theta + 4 * j));
    g[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p.grad + 4 * j));
    m[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p.m + 4 * j));
    v[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p.v + 4 * j));
  }
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    if (idx[i] >= p.nvec) continue;
    float t4[4], m4[4], v4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      t4[q] = th[i][q];
      m4[q] = m[i][q];
      v4[q] = v[i][q];
      adamw_elem(p, t4[q], g[i][q], m4[q], v4[q]);
    }
    const int64_t o = 4 * idx[i];
    __builtin_nontemporal_store(f32x4_t{t4[0], t4[1], t4[2], t4[3]}, reinterpret_cast<f32x4_t *>(p.theta + o));
    __builtin_nontemporal_store(f32x4_t{m4[0], m4[1], m4[2], m4[3]}, reinterpret_cast<f32x4_t *>(p.m + o));
    __builtin_nontemporal_store(f32x4_t{v4[0], v4[1], v4[2], v4[3]}, reinterpret_cast<f32x4_t *>(p.v + o));
    if (p.lowp) {
      typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
      __builtin_nontemporal_store(u32x2_t{pack_bf2(t4[0], t4[1]), pack_bf2(t4[2], t4[3])},
                                  reinterpret_cast<u32x2_t *>(p.lowp + o));
    }
    if (p.zero_grad) __builtin_nontemporal_store(f32x4_t{0.f, 0.f, 0.f, 0.f}, reinterpret_cast<f32x4_t *>(p.grad + o));
  }
}

// The last n % 4 elements, one thread each.
__global__ void adamw_tail_kernel(AdamwParams p, int64_t first, int count) {
  const int i = threadIdx.x;
  if (i >= count) return;
  const int64_t e = first + i;
  float th = p.theta[e], m = p.m[e], v = p.v[e];
  adamw_elem(p, th, p.grad[e], m, v);
  p.theta[e] = th;
  p.m[e] = m;
  p.v[e] = v;
  if (p.lowp) p.lowp[e] = f2bf(th);
  if (p.zero_grad) p.grad[e] = 0.f;
}

hipError_t launch_adamw(const AdamwLaunch &a, hipStream_t s) {
  LaunchScope scope("adamw", s);
  AdamwParams p;
  p.theta = a.theta;
  p.grad = a.grad;
  p.m = a.m;
  p.v = a.v;
  p.lowp = (bf16_t *)a.lowp;
  p.nvec = a.n / 4;
  p.b1 = a.b1;
  p.b2 = a.b2;
  p.one_minus_b1 = 1.f - a.b1;
  p.one_minus_b2 = 1.f - a.b2;
  p.decay = a.decay;
  p.step_size = a.step_size;
  p.bc2_sqrt = a.bc2_sqrt;
  p.eps = a.eps;
  p.scale = a.scale;
  p.zero_grad = a.zero_grad ? 1 : 0;
  if (p.nvec > 0) {
    const int64_t per_block = (int64_t)kAdamThreads * kVecPerThread;
    const unsigned grid = (unsigned)((p.nvec + per_block - 1) / per_block);
    adamw_kernel<<<grid, kAdamThreads, 0, s>>>(p);
  }
  const int tail = (int)(a.n - 4 * p.nvec);
  if (tail > 0) adamw_tail_kernel<<<1, 64, 0, s>>>(p, 4 * p.nvec, tail);
  return hipGetLastError();
}

}  // namespace moe
