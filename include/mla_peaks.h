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

/* Cycle cost of 32x32x16 bf16 MFMAs issued by one wavefront per SIMD
 * (`groups` workgroups of 256 threads; at 256 groups one per compute unit):
 * each wavefront runs `iters` rounds of `chains` (1 or 2) accumulator chains,
 * every MFMA followed by `valu_per_mfma` (0, 2, 4, 6, 8 or 12) independent
 * fp32 FMAs.  cycles holds 2 * groups entries: per workgroup the shader-clock
 * cycles (s_memtime) and the 100 MHz reference ticks (s_memrealtime) of the
 * loop, so cycles per MFMA = cycles / (iters * chains) and the shader clock =
 * cycles / ticks * 100 MHz.  sink holds groups * 256 floats, written only for
 * an unlikely value.  Other chain or VALU counts return hipErrorInvalidValue. */
int32_t peak_mfma_cycles(int32_t groups, int32_t iters, int32_t chains, int32_t valu_per_mfma,
                         uint64_t* cycles, float* sink, void* stream);

/* LDS bandwidth: `groups` workgroups of 256 * waves_per_simd threads (1 or 2
 * wavefronts per SIMD), each holding 64 KiB of LDS; every thread reads
 * (write = 0) or writes (write != 0) 8 conflict-free words of `width` bytes
 * (4, 8 or 16: ds_read/ds_write _b32, _b64, _b128) per round, `iters`
 * rounds.  cycles[g] = shader-clock cycles of workgroup g's loop, so bytes
 * per cycle per compute unit = iters * 8 * width * threads / cycles when one
 * workgroup runs per compute unit.  sink holds groups * 256 * waves_per_simd
 * words, written only for an unlikely value.  Invalid arguments return
 * hipErrorInvalidValue before any launch. */
int32_t peak_lds(int32_t groups, int32_t waves_per_simd, int32_t write, int32_t width, int32_t iters,
                 uint64_t* cycles, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif
