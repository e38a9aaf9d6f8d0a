/*
 * qkra_calibrate -- roofline calibration kernels for the benchmark of the
 * attention library (not part of the attention path): how fast this MI355X
 * streams a buffer from HBM and how many bf16 matrix-core operations per
 * second it sustains, so that the attention kernels' rates can be stated
 * against what is reachable on this part as well as against the published
 * peaks.  The concept chapter "Chapter 3 Forward Pass and Generation",
 * section 4.3, splits the work into compute-bound prefill and
 * bandwidth-bound decode: these are the two ceilings.
 *
 * Built as its own shared library, libqkra_calibrate.so.  All pointers are
 * DEVICE pointers owned by the caller; work goes onto `hip_stream` (a
 * hipStream_t, NULL = the default stream) without synchronising.  Return
 * value 0 = enqueued, 1 = invalid argument (nothing enqueued), 6 = the
 * launch failed.
 */
#ifndef QKRA_CALIBRATE_H
#define QKRA_CALIBRATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKRA_CALIB_API __attribute__((visibility("default")))

/*
 * Reads `bytes` (a multiple of 16) of `buf` (16-byte aligned) once, with
 * 16-byte non-temporal loads from `workgroups` workgroups of 256 threads:
 * each wavefront streams a contiguous share, 1 KB per load instruction, eight
 * instructions in flight.  `sink` (4 bytes) is never written in
 * practice; it keeps the loads alive.  Rate = bytes / kernel time.  Use a
 * buffer well above the 256 MB last-level cache.
 */
QKRA_CALIB_API int32_t qkra_calibrate_stream_read(const void* buf, size_t bytes, void* sink,
                                                  int32_t workgroups, void* hip_stream);

/*
 * Copies `bytes` (a multiple of 16) from `src` to `dst` (both 16-byte aligned,
 * not overlapping: 1 otherwise): one 16-byte piece per thread, non-temporal
 * load and store, 256 threads per workgroup, as many workgroups as pieces.
 * Rate = 2 * bytes / kernel time (bytes read plus bytes written).
 */
QKRA_CALIB_API int32_t qkra_calibrate_stream_copy(const void* src, void* dst, size_t bytes, void* hip_stream);

/*
 * `workgroups` workgroups of 4 wavefronts (two per SIMD when there are two
 * per CU), each running `iterations` rounds of four independent
 * v_mfma_f32_32x32x16_bf16 on register operands.  `sink` (workgroups floats)
 * is never written in practice.  Rate = qkra_calibrate_mfma_flop(iterations,
 * workgroups) / kernel time.
 */
QKRA_CALIB_API int32_t qkra_calibrate_mfma_bf16(int64_t iterations, void* sink, int32_t workgroups,
                                                void* hip_stream);
QKRA_CALIB_API size_t qkra_calibrate_mfma_flop(int64_t iterations, int32_t workgroups);

#ifdef __cplusplus
}
#endif

#endif /* QKRA_CALIBRATE_H */
