// Append kernel: quantize + pack + write new MLA cache rows into paged
// storage (the row arithmetic is in append.h).
//
// Launch: one wavefront per token, 4 tokens per 256-thread workgroup; rows
// whose slot is negative or beyond the pool are skipped.
#include "append.h"
#include "kernels.h"

namespace mla {

template <int F>
__global__ __launch_bounds__(256) void k_quant_append(const __bf16* __restrict__ latent,
                                                      const __bf16* __restrict__ rope,
                                                      const int32_t* __restrict__ slots, int n_new,
                                                      uint8_t* __restrict__ cache, int64_t num_pages) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= n_new) return;
  const int slot = slots[n];
  if (slot < 0) return;
  const int64_t page = slot / kPage;
  if (page >= num_pages) return;
  append_row<F>(latent + (int64_t)n * kDc, rope + (int64_t)n * kDr, cache + page * (int64_t)PageLayout<F>::kBytes,
                slot % kPage);
}

hipError_t launch_quant_append(int fmt, const void* latent, const void* rope, const int32_t* slots,
                               int n_new, void* cache, int64_t num_pages, hipStream_t stream) {
  const dim3 grid((n_new + 3) / 4), block(256);
  const __bf16* l = (const __bf16*)latent;
  const __bf16* r = (const __bf16*)rope;
  uint8_t* c = (uint8_t*)cache;
  if (fmt == kC4R4) hipLaunchKernelGGL(k_quant_append<kC4R4>, grid, block, 0, stream, l, r, slots, n_new, c, num_pages);
  else if (fmt == kC2R4) hipLaunchKernelGGL(k_quant_append<kC2R4>, grid, block, 0, stream, l, r, slots, n_new, c, num_pages);
  else hipLaunchKernelGGL(k_quant_append<kBF16>, grid, block, 0, stream, l, r, slots, n_new, c, num_pages);
  return hipGetLastError();
}

}  // namespace mla
