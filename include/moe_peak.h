/*
 * moe_peak.h -- attainable-peak probes of the MoE library, for measurement.
 *
 * Not part of the layer: these give the rates the layer's kernels are set
 * against beside MI355X's published peaks (2.5 PFLOP/s dense bf16 MFMA,
 * 8 TB/s HBM3E), measured on the GPU they run on.
 */
#ifndef MOE_MI355X_PEAK_H
#define MOE_MI355X_PEAK_H

#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * bf16 matrix-core loop: two workgroups of four wavefronts per compute unit,
 * each wavefront issuing v_mfma_f32_32x32x16_bf16 (the grouped GEMMs'
 * instruction) `iters` times on each of four independent fp32 accumulators
 * from register operands; no memory traffic but one fp32 per thread written
 * to `out` at the end. out: device buffer of at least moe_peak_mfma_size()
 * floats (16-byte aligned). *flops receives the FLOPs the launch performs
 * (2*32*32*16 per wavefront and instruction). Asynchronous on `stream`; the
 * caller times it. Errors: out or flops NULL, iters < 1 ->
 * MOE_ERR_INVALID_ARGUMENT; a misaligned out -> MOE_ERR_MISALIGNED.
 */
moe_status moe_peak_mfma(float *out, int32_t iters, double *flops, moe_stream_t stream);

/* Floats `out` of moe_peak_mfma must hold on the current device. */
int64_t moe_peak_mfma_size(void);

/*
 * Plain device copy of `bytes` bytes from src to dst (one 16-byte
 * non-temporal load and store per thread, one launch): 2*bytes of HBM
 * traffic when the buffers exceed the caches. bytes must be a positive
 * multiple of 16, src and dst 16-byte aligned and not overlapping.
 * Asynchronous on `stream`.
 */
moe_status moe_peak_copy(const void *src, void *dst, int64_t bytes, moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_PEAK_H */
