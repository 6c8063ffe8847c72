// Attainable-peak probes for the measurement (not part of the layer): the
// rate the matrix cores reach on the instruction the grouped GEMMs use, and
// the rate a plain device copy reaches in HBM. The bench reports the layer's
// kernels against these beside the published peaks.
#include "common.h"
#include "kernels.h"

namespace moe {

// Every wavefront keeps NACC independent 32x32 fp32 accumulators and issues
// v_mfma_f32_32x32x16_bf16 on them in turn from register operands, so nothing
// but the matrix cores bounds the loop. Each thread stores one sum at the end
// so that no accumulator is dead.
template <int NACC>
__global__ __launch_bounds__(256) void peak_mfma_kernel(float *__restrict__ out, int iters) {
  const int tid = threadIdx.x;
  f32x16_t acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
  bf16x8_t a, b;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    a[q] = (__bf16)((float)((tid + q) & 7) * 0.125f);
    b[q] = (__bf16)((float)((tid * 3 + q) & 7) * 0.0625f);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NACC; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[i][v];
  out[(int64_t)blockIdx.x * blockDim.x + tid] = s;
}

// One 16-byte chunk per thread, consecutive lanes on consecutive chunks, one
// launch over the whole buffer, every byte touched once (non-temporal load
// and store). Of the copy forms measured on MI355X (grid-stride loops, 2-8
// chunks per thread, cached accesses, the runtime's device copy) this one
// streams fastest.
__global__ __launch_bounds__(256) void peak_copy_kernel(const u32x4_t *__restrict__ src, u32x4_t *__restrict__ dst,
                                                        int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) st16_nt(dst + i, ld16_nt(src + i));
}

constexpr int kPeakAcc = 4;

int peak_mfma_threads(int cus) { return cus * 2 * 256; }

double peak_mfma_flops(int cus, int iters) {
  // 64 lanes share one 32x32x16 product: 2*32*32*16 FLOP per wavefront issue
  const double waves = (double)peak_mfma_threads(cus) / 64.0;
  return waves * (double)iters * kPeakAcc * 2.0 * 32 * 32 * 16;
}

hipError_t launch_peak_mfma(float *out, int cus, int iters, hipStream_t s) {
  LaunchScope scope("peak_mfma", s);
  // two 4-wavefront workgroups per CU: two wavefronts per SIMD, each with
  // kPeakAcc independent accumulator chains
  peak_mfma_kernel<kPeakAcc><<<dim3((unsigned)(cus * 2)), 256, 0, s>>>(out, iters);
  return hipGetLastError();
}

hipError_t launch_peak_copy(const void *src, void *dst, int64_t bytes, hipStream_t s) {
  LaunchScope scope("peak_copy", s);
  const int64_t n16 = bytes / 16;
  peak_copy_kernel<<<dim3((unsigned)((n16 + 255) / 256)), 256, 0, s>>>((const u32x4_t *)src, (u32x4_t *)dst, n16);
  return hipGetLastError();
}

}  // namespace moe
