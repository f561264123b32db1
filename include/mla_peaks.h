/* Microbenchmarks that measure the practical peaks the decode kernels are
 * compared with on gfx950 (libmla_peaks.so; separate from the decode
 * library).  All pointers are device pointers owned by the caller; every
 * call is asynchronous on `stream` (a hipStream_t, NULL for the default
 * stream) and returns 0 on success or the HIP error code of the launch.
 * Nothing here allocates or synchronises. */
#ifndef MLA_PEAKS_H
#define MLA_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Plain copy of `bytes` (a multiple of 16, both pointers 16-byte aligned):
 * reads exactly `bytes` and writes exactly `bytes`.  It is the reference of
 * known size for the HBM byte counters (FETCH_SIZE / WRITE_SIZE). */
int32_t peak_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Streaming read of `bytes` (a multiple of 16384, 16-byte aligned) with
 * `groups` workgroups of 256 threads; the loaded data is folded into one
 * word that is stored to sink[0] only if it equals a fixed unlikely value
 * (so the loads cannot be removed). */
int32_t peak_read(const void* src, size_t bytes, int32_t groups, uint32_t* sink, void* stream);

/* Dense bf16 MFMA loop: `groups` workgroups of 256 threads, each wavefront
 * issuing `iters` rounds of 4 independent 32x32x16 bf16 MFMAs (fp32
 * accumulate).  Flops = groups * 4 * iters * 4 * 32768.  sink holds
 * groups * 256 floats, written only for an unlikely accumulator value. */
int32_t peak_mfma_bf16(int32_t groups, int32_t iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif
