// The absorbed projections on either side of the decode (one MLA decode
// attention step).  MLA keeps one latent per token as the shared source of
// keys and values ("QuantMLA: INT4 (and INT2) for both halves of the MLA
// cache", TL;DR and flowchart): head h's key is W_UK[h] c and its value
// W_UV[h] c.  Decode never forms them: the query is absorbed into latent
// space before attention (q_c = W_UK[h]^T q_nope) and the value projection is
// applied once to the attention result after it (o = W_UV[h] out).
//
// Both are per-head GEMMs  y[b, h, n] = sum_k x[b, h, k] w[h, n, k]  (fp32
// accumulate, bf16 round-to-nearest-even output) on MFMA 32x32x16 bf16:
//   absorb:  x = q_nope [B, H, 128], w = W_UK [H, 512, 128] -> q[b, h, 0:512]
//            (and q[b, h, 512:576] = q_pe[b, h, :]), q row stride 576
//   output:  x = out [B, H, 512],    w = W_UV [H, 128, 512] -> o [B, H, 128]
// Weights are stored n-major (w[h][n][k], k contiguous) so both MFMA operands
// are 16-byte row loads; the decode batch is the M dimension (rows >= B are
// zero).  The work is bound by reading the weights once.
#include "kernels.h"

namespace mla {

constexpr int kProjThreads = 256;

// Workgroup (h, part): n-blocks [part * NBW, (part + 1) * NBW) of head h, all
// row blocks; the 4 wavefronts take (row block, n-block) items in turn.
template <int K>
__global__ __launch_bounds__(kProjThreads) void k_head_gemm(const __bf16* __restrict__ x, const __bf16* __restrict__ w,
                                                            int B, int H, int N, int nbw, __bf16* __restrict__ y,
                                                            int y_stride, const __bf16* __restrict__ tail,
                                                            int tail_len) {
  const int h = blockIdx.x, part = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int mrow = lane & 31, khalf = lane >> 5;
  const int mblocks = (B + 31) / 32;
  const __bf16* wh = w + (int64_t)h * N * K;
  for (int item = wave; item < mblocks * nbw; item += kProjThreads / 64) {
    const int mb = item / nbw, nb = part * nbw + item % nbw;
    const int b = mb * 32 + mrow;
    const __bf16* xr = x + ((int64_t)(b < B ? b : 0) * H + h) * K + 8 * khalf;
    const __bf16* wr = wh + (int64_t)(nb * 32 + mrow) * K + 8 * khalf;
    const bf16x8 zero = {};
    f32x16 acc = {};
#pragma unroll 8
    for (int ks = 0; ks < K / 16; ++ks) {
      const bf16x8 av = b < B ? *(const bf16x8*)(xr + 16 * ks) : zero;
      const bf16x8 bv = *(const bf16x8*)(wr + 16 * ks);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
    }
    // D layout: reg r holds row 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32
    const int n = nb * 32 + mrow;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int bo = mb * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
      if (bo < B) y[((int64_t)bo * H + h) * y_stride + n] = (__bf16)acc[r];
    }
  }
  // the absorbed query's RoPE part is the input's, copied after the latent part
  if (tail && part == 0)
    for (int i = threadIdx.x; i < B * tail_len; i += kProjThreads) {
      const int b = i / tail_len, j = i % tail_len;
      y[((int64_t)b * H + h) * y_stride + N + j] = tail[((int64_t)b * H + h) * tail_len + j];
    }
}

hipError_t launch_absorb_q(const void* q_nope, const void* q_pe, const void* w_uk, int B, int H, void* q_out,
                           hipStream_t stream) {
  // N = 512: 16 n-blocks, one per wavefront: four workgroups per head
  hipLaunchKernelGGL(k_head_gemm<128>, dim3(H, 4), dim3(kProjThreads), 0, stream, (const __bf16*)q_nope,
                     (const __bf16*)w_uk, B, H, kDc, 4, (__bf16*)q_out, kD, (const __bf16*)q_pe, kDr);
  return hipGetLastError();
}

hipError_t launch_project_out(const void* latent, const void* w_uv, int B, int H, void* out, hipStream_t stream) {
  // N = 128: 4 n-blocks, two workgroups per head
  hipLaunchKernelGGL(k_head_gemm<kDc>, dim3(H, 2), dim3(kProjThreads), 0, stream, (const __bf16*)latent,
                     (const __bf16*)w_uv, B, H, 128, 2, (__bf16*)out, 128, (const __bf16*)nullptr, 0);
  return hipGetLastError();
}

}  // namespace mla
