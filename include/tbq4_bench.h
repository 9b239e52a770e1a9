/*
 * tbq4_bench.h -- measurement helpers of libtbq4 (not attention calls).
 *
 * The roofline fractions of the attention kernels are reported against the
 * part's published peaks and against what the part measurably sustains on
 * the same kind of work: these two calls provide the latter.  Neither takes
 * part in the attention hot path; both only read their inputs and write a
 * sink the caller discards.
 *
 * tbq4_bench_stream_read: n_blocks workgroups of 256 threads read `bytes`
 *   bytes at `buf` (device, 16-byte aligned, bytes a multiple of 16) once,
 *   16 bytes per lane per load with non-temporal hints, four loads in flight
 *   per lane; every workgroup writes one uint32 to sink[blockIdx] (device,
 *   n_blocks words).  Achievable read bandwidth = bytes / kernel time.
 * tbq4_bench_mfma_f16: n_blocks workgroups of 4 wavefronts each issue
 *   iters x 8 independent v_mfma_f32_32x32x16_f16 (32768 flops each) on
 *   register operands; every thread writes one float to sink (device,
 *   n_blocks * 256 floats).  Achievable dense fp16 MFMA rate = n_blocks * 4 *
 *   iters * 8 * 32768 flops / kernel time.
 * Both enqueue one launch on hip_stream and return 0, -1 for a bad argument
 * or -6 when the HIP runtime reports a launch error.
 */
#ifndef TBQ4_BENCH_H
#define TBQ4_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t tbq4_bench_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t n_blocks,
                               void *hip_stream);
int32_t tbq4_bench_mfma_f16(int32_t iters, float *sink, int32_t n_blocks, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* TBQ4_BENCH_H */
