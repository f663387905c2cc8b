/*
 * Measured machine ceilings for the benchmark's context figures.
 *
 * These calls are not part of the codec.  They run plain streaming and
 * arithmetic loops on the caller's stream so that the benchmark can put each
 * codec kernel beside what this particular GPU delivers (the published
 * MI355X peaks stay the contract; these are context).  The caller times them
 * with events on the same stream.
 *
 * Error codes are those of hqmq.h (HQMQ_OK, HQMQ_EINVAL, HQMQ_EHIP).
 */
#ifndef HQMQ_CEILING_H
#define HQMQ_CEILING_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    HQMQ_CEIL_READ = 0,   /* read src once (bytes read) */
    HQMQ_CEIL_WRITE = 1,  /* write dst once, non-temporal 16-byte stores (bytes written) */
    HQMQ_CEIL_COPY = 2    /* copy src to dst (bytes read + bytes written) */
};

/* One streaming pass over `bytes` bytes, shaped like the codec's
 * bandwidth-bound kernels: each thread has 8 independent 16-byte accesses in
 * flight and each access instruction of a wave covers 1 KB of consecutive
 * bytes (non-temporal loads and stores).  src and dst are device pointers,
 * 16-byte aligned; bytes is a positive multiple of 16 (src is unused for
 * WRITE, dst is unused for READ except for one 4-byte word that keeps the
 * read live; the caller owns both).  Asynchronous on `stream`.
 * Returns HQMQ_EINVAL on a bad kind, size or alignment (nothing enqueued),
 * HQMQ_EHIP if the launch fails. */
int hqmq_ceiling_stream(int kind, const void *src, void *dst, size_t bytes, hipStream_t stream);

enum {
    HQMQ_CEIL_FMA_F32 = 0,   /* v_fma_f32, 16 independent chains per lane */
    HQMQ_CEIL_MFMA_F32 = 1,  /* v_mfma_f32_16x16x4f32, 4 independent accumulators per wave */
    HQMQ_CEIL_MFMA_F16 = 2   /* v_mfma_f32_32x32x8_f16, 2 independent accumulators per wave */
};

/* An arithmetic loop of `iterations` rounds on every SIMD of the device
 * (8 waves per SIMD).  *flops receives the floating-point operations the
 * launch performs (an FMA or a multiply-add in a matrix product counts 2).
 * `sink` is a device float the loop's result may be written to (so the loop
 * is not removed); the caller owns it.  Asynchronous on `stream`.
 * Returns HQMQ_EINVAL on a bad kind or iterations < 1 (nothing enqueued),
 * HQMQ_EHIP if the launch or the device query fails. */
int hqmq_ceiling_compute(int kind, int64_t iterations, float *sink, hipStream_t stream, double *flops);

#ifdef __cplusplus
}
#endif

#endif /* HQMQ_CEILING_H */
