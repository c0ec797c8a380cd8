/*
 * swan_measure.h -- measurement helpers of libswan, beside the decode step's
 * entry points (swan.h).  They compute nothing of the method: they give the
 * yardsticks its kernels are measured against on the GPU they run on.
 *
 * The SWAN page's background on autoregressive generation notes that a
 * decode step reads the whole KV cache from HBM for one query, so the step
 * is bound by memory bandwidth.  The ceiling a decode kernel can reach is
 * then what a plain streaming read of the same number of bytes achieves on
 * the same GPU, below the published peak.
 *
 * The prefill conversion projects every key of a history through P_QK in
 * double precision, a dense contraction that runs on the fp64 matrix
 * cores; its ceiling is the rate those cores sustain on independent
 * products.
 */
#ifndef SWAN_MEASURE_H
#define SWAN_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "swan.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * A streaming read of `bytes` bytes at `buf` (device, 16-byte aligned,
 * bytes a multiple of 16), in `waves` one-wave workgroups (1..1048576) that
 * each read one contiguous share with 16-byte non-temporal loads, eight in
 * flight a lane.  Every loaded word is folded (xor) into sink[wave * 64 +
 * lane] (device, waves * 64 uint32 written), so no load can be dropped.
 * Asynchronous on `stream`; the caller times it (e.g. with events around
 * back-to-back launches).  Errors: SWAN_ERR_INVALID_ARG for NULL pointers,
 * a misaligned buffer, bytes not a multiple of 16 or zero, or waves outside
 * 1..1048576 (nothing is launched); SWAN_ERR_HIP for a failed launch.
 */
swan_status swan_measure_stream_read(const void *buf, size_t bytes, int32_t waves, uint32_t *sink, void *stream);

/*
 * fp64 matrix-core rate: `waves` waves (1..1048576, in workgroups of four)
 * each run `iters` (a multiple of 4 in 4..1048576) rounds of eight
 * independent v_mfma_f64_16x16x4f64 products (2 x 16 x 16 x 4 flops each,
 * so 16384 flops a wave a round) with every A and B element equal to x, and
 * write the sum of the lane's accumulator elements to sink[wave * 64 +
 * lane] (device, waves * 64 doubles): 128 x^2 iters when no rounding occurs
 * (x = 1).  Asynchronous on `stream`; the caller times it.  Errors:
 * SWAN_ERR_INVALID_ARG for a NULL sink or waves / iters out of range
 * (nothing is launched); SWAN_ERR_HIP for a failed launch.
 */
swan_status swan_measure_mfma_f64(double x, int32_t waves, int32_t iters, double *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SWAN_MEASURE_H */
