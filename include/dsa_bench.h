/*
 * dsa_bench.h - on-device peak measurements for the MI355X (gfx950) figures the indexer
 * kernels are rated against.
 *
 * The scoring kernel is a dense contraction on the matrix cores, and the preprocessing
 * and top-k kernels stream HBM. Their rates are reported against the published MI355X
 * peaks (dense MFMA: 2.5 PFLOP/s bf16, 5.0 PFLOP/s fp8; HBM3E 8 TB/s) and against what
 * the device in hand sustains, measured by these two calls: a compute-only stream of the
 * scoring kernel's MFMA instruction, and a sweep over a device buffer. They are measurement
 * helpers, not part of the indexer's method. Conventions as in dsa_index.h: device pointers
 * owned by the caller, host scalars, asynchronous on `stream`, a status return with
 * dsa_last_error() describing a non-OK status, nothing allocated or synchronised.
 */
#ifndef DSA_BENCH_H
#define DSA_BENCH_H

#include "dsa_index.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * dsa_bench_mfma - `blocks` workgroups of 256 threads (4 waves) each run `iters` rounds of
 * four independent accumulator chains of one MFMA instruction, operands in registers:
 *   DSA_PREC_BF16            v_mfma_f32_32x32x16_bf16     (32768 flops per instruction)
 *   DSA_PREC_FP8, _MXFP8     v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E4M3, unit scales
 *                                                         (131072 flops per instruction)
 *   out     device float [blocks * 256]: one sum of accumulators per thread (written so the
 *           work is kept; the values carry no meaning).
 * The flops of one call are dsa_bench_mfma_flops(precision, blocks, iters); time the call
 * with events on `stream`.
 * Errors: DSA_ERR_UNSUPPORTED for an unknown precision; DSA_ERR_INVALID_ARGUMENT for
 * blocks or iters < 1, blocks > 65536, or out NULL or not 4-byte aligned; DSA_ERR_DEVICE
 * on a launch error.
 */
dsa_status_t dsa_bench_mfma(dsa_precision_t precision, int32_t blocks, int32_t iters, float* out,
                            hipStream_t stream);
double dsa_bench_mfma_flops(dsa_precision_t precision, int32_t blocks, int32_t iters);

/*
 * dsa_bench_stream - a sweep over `bytes` of src in 16-byte vectors (grid-stride, four loads
 * in flight per thread, at most 8192 workgroups of 256 threads).
 *   copy = 1: every vector is written to dst (dst holds `bytes`); HBM traffic 2 * bytes.
 *   copy = 0: read only (dst holds at least 16 bytes and is in practice never written);
 *             HBM traffic `bytes`.
 * Errors: DSA_ERR_INVALID_ARGUMENT for bytes 0 or not a multiple of 16, src or dst NULL or
 * not 16-byte aligned, copy not 0 or 1; DSA_ERR_DEVICE on a launch error.
 */
dsa_status_t dsa_bench_stream(const void* src, void* dst, size_t bytes, int32_t copy, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_BENCH_H */
