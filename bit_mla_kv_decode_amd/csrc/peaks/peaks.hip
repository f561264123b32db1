// Practical-peak microbenchmarks for gfx950: streaming HBM read, plain copy
// (the reference for HBM byte counters), a dense bf16 MFMA loop, the cycle
// cost of MFMA chains with VALU work between them, and LDS bandwidth.
#include <hip/hip_runtime.h>

#include "mla_peaks.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void k_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// four 16-byte loads in flight per thread per round
__global__ __launch_bounds__(256) void k_read(const u32x4* __restrict__ src, int64_t n4, unsigned* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  u32x4 acc = {};
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const u32x4* p = src + 4 * (i - threadIdx.x) + threadIdx.x;
    const u32x4 a = __builtin_nontemporal_load(p);
    const u32x4 b = __builtin_nontemporal_load(p + 256);
    const u32x4 c = __builtin_nontemporal_load(p + 512);
    const u32x4 d = __builtin_nontemporal_load(p + 768);
    acc ^= a ^ b ^ c ^ d;
  }
  const unsigned v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (v == 0x9e3779b9u) sink[0] = v;
}

__global__ __launch_bounds__(256) void k_mfma(int iters, float* __restrict__ sink) {
  const int t = threadIdx.x;
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)((t + e) & 7);
    b[e] = (__bf16)(float)((t * 3 + e) & 7);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (s == -1.0f) sink[(int64_t)blockIdx.x * 256 + t] = s;
}


// MFMA issue cost in shader cycles.  One wavefront per SIMD (256 threads per
// workgroup, one workgroup per compute unit at 256 workgroups): `iters`
// rounds of CH accumulator chains of 32x32x16 bf16 MFMAs, each MFMA followed
// by NV fp32 FMAs on registers the MFMAs do not touch; scheduling barriers
// keep that order.  Operands vary per lane so the data toggles like real
// data.  Thread 0 stores the s_memtime and s_memrealtime (100 MHz) deltas.
template <int CH, int NV>
__global__ __launch_bounds__(256) void k_mfma_cycles(int iters, unsigned long long* __restrict__ cycles,
                                                     float* __restrict__ sink) {
  const int t = threadIdx.x;
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)((float)((t * 7 + e * 13) % 97) * 0.0173f - 0.8f);
    b[e] = (__bf16)((float)((t * 5 + e * 11) % 89) * 0.0191f - 0.7f);
  }
  f32x16 c[CH];
  for (int j = 0; j < CH; ++j) c[j] = (f32x16){};
  float v[16];
  for (int j = 0; j < 16; ++j) v[j] = (float)(t + j);
  const float m = 1.0001f, d = 0.5f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < NV; ++k) v[(8 * j + k) & 15] = __builtin_fmaf(v[(8 * j + k) & 15], m, d);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = 0.0f;
  for (int j = 0; j < CH; ++j)
    for (int e = 0; e < 16; ++e) s += c[j][e];
  for (int e = 0; e < 16; ++e) s += v[e];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (t == 0) {
    cycles[2 * blockIdx.x] = t1 - t0;
    cycles[2 * blockIdx.x + 1] = r1 - r0;
  }
  if (s == -1.0f) sink[(int64_t)blockIdx.x * 256 + t] = s;
}

// LDS bandwidth: each workgroup holds 64 KiB of LDS (at most two per compute
// unit); thread t reads (or writes) W bytes (W = 4, 8 or 16) at t W + 4096 j
// + 16 (i & 1), j < 8 (consecutive lanes on consecutive words: no bank
// conflicts; all inside the first 45 KiB), `iters` times.  Thread 0 stores
// the s_memtime delta of the loop.
template <int W, bool WRITE>
__global__ __launch_bounds__(512) void k_lds(int iters, unsigned long long* __restrict__ cycles,
                                             unsigned* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[65536];
  const int t = threadIdx.x;
  for (int i = t; i < 65536 / 16; i += blockDim.x) ((u32x4*)lds)[i] = (u32x4){(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      unsigned char* p = lds + t * W + j * 4096 + 16 * (it & 1);
      if (WRITE) {
        const u32x4 v = acc + (u32x4){(unsigned)it, 0u, 0u, 0u};
        if (W == 4) *(unsigned*)p = v.x;
        if (W == 8) *(u32x2*)p = (u32x2){v.x, v.y};
        if (W == 16) *(u32x4*)p = v;
      } else {
        if (W == 4) acc.x ^= *(const unsigned*)p;
        if (W == 8) {
          const u32x2 r = *(const u32x2*)p;
          acc.x ^= r.x;
          acc.y ^= r.y;
        }
        if (W == 16) acc ^= *(const u32x4*)p;
      }
    }
    asm volatile("" ::"v"(lds) : "memory");  // the array escapes: every store stays
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (t == 0) cycles[blockIdx.x] = t1 - t0;
  acc ^= *(const u32x4*)(lds + 16 * ((t + 1) % blockDim.x));
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x12345678u) sink[(int64_t)blockIdx.x * blockDim.x + t] = acc.x;
}

template <int W>
hipError_t launch_lds(bool write, int groups, dim3 block, int iters, unsigned long long* cycles, unsigned* sink,
                      hipStream_t st) {
  if (write)
    hipLaunchKernelGGL((k_lds<W, true>), dim3(groups), block, 0, st, iters, cycles, sink);
  else
    hipLaunchKernelGGL((k_lds<W, false>), dim3(groups), block, 0, st, iters, cycles, sink);
  return hipGetLastError();
}

template <int CH>
hipError_t launch_mfma_cycles(int nv, int groups, int iters, unsigned long long* cycles, float* sink, hipStream_t st) {
  switch (nv) {
    case 0: hipLaunchKernelGGL((k_mfma_cycles<CH, 0>), dim3(groups), dim3(256), 0, st, iters, cycles, sink); break;
    case 2: hipLaunchKernelGGL((k_mfma_cycles<CH, 2>), dim3(groups), dim3(256), 0, st, iters, cycles, sink); break;
    case 4: hipLaunchKernelGGL((k_mfma_cycles<CH, 4>), dim3(groups), dim3(256), 0, st, iters, cycles, sink); break;
    case 6: hipLaunchKernelGGL((k_mfma_cycles<CH, 6>), dim3(groups), dim3(256), 0, st, iters, cycles, sink); break;
    case 8: hipLaunchKernelGGL((k_mfma_cycles<CH, 8>), dim3(groups), dim3(256), 0, st, iters, cycles, sink); break;
    case 12: hipLaunchKernelGGL((k_mfma_cycles<CH, 12>), dim3(groups), dim3(256), 0, st, iters, cycles, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int32_t status(hipError_t e) { return e == hipSuccess ? 0 : (int32_t)e; }

}  // namespace

extern "C" {

int32_t peak_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes % 16 || (uintptr_t)src % 16 || (uintptr_t)dst % 16) return (int32_t)hipErrorInvalidValue;
  if (bytes == 0) return 0;
  const int64_t n = (int64_t)(bytes / 16);
  const int64_t want = (n + 255) / 256;
  const int groups = (int)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(k_copy, dim3(groups), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, (u32x4*)dst, n);
  return status(hipGetLastError());
}

int32_t peak_read(const void* src, size_t bytes, int32_t groups, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes % 16384 || (uintptr_t)src % 16 || groups < 1) return (int32_t)hipErrorInvalidValue;
  // k_read walks blocks of 4 * 256 16-byte vectors (16 KiB)
  const int64_t n4 = (int64_t)(bytes / 16384) * 256;
  if (n4 == 0) return 0;
  hipLaunchKernelGGL(k_read, dim3(groups), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, n4, sink);
  return status(hipGetLastError());
}

int32_t peak_mfma_bf16(int32_t groups, int32_t iters, float* sink, void* stream) {
  if (!sink || groups < 1 || iters < 0) return (int32_t)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mfma, dim3(groups), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return status(hipGetLastError());
}

int32_t peak_mfma_cycles(int32_t groups, int32_t iters, int32_t chains, int32_t valu_per_mfma,
                         uint64_t* cycles, float* sink, void* stream) {
  if (!cycles || !sink || groups < 1 || iters < 0) return (int32_t)hipErrorInvalidValue;
  hipError_t e;
  if (chains == 1)
    e = launch_mfma_cycles<1>(valu_per_mfma, groups, iters, (unsigned long long*)cycles, sink, (hipStream_t)stream);
  else if (chains == 2)
    e = launch_mfma_cycles<2>(valu_per_mfma, groups, iters, (unsigned long long*)cycles, sink, (hipStream_t)stream);
  else
    return (int32_t)hipErrorInvalidValue;
  return status(e);
}

int32_t peak_lds(int32_t groups, int32_t waves_per_simd, int32_t write, int32_t width, int32_t iters,
                 uint64_t* cycles, uint32_t* sink, void* stream) {
  if (!cycles || !sink || groups < 1 || iters < 0 || (waves_per_simd != 1 && waves_per_simd != 2) ||
      (width != 4 && width != 8 && width != 16))
    return (int32_t)hipErrorInvalidValue;
  const dim3 block(256 * waves_per_simd);
  unsigned long long* c = (unsigned long long*)cycles;
  const hipStream_t st = (hipStream_t)stream;
  const hipError_t e = width == 4   ? launch_lds<4>(write != 0, groups, block, iters, c, sink, st)
                       : width == 8 ? launch_lds<8>(write != 0, groups, block, iters, c, sink, st)
                                    : launch_lds<16>(write != 0, groups, block, iters, c, sink, st);
  return status(e);
}

}  // extern "C"
