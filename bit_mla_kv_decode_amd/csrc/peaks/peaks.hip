// Practical-peak microbenchmarks for gfx950: streaming HBM read, plain copy
// (the reference for HBM byte counters) and a dense bf16 MFMA loop.
#include <hip/hip_runtime.h>

#include "mla_peaks.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
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

}  // extern "C"
