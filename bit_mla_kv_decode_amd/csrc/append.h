// Quantize + pack one new MLA cache row (per token: content latent and RoPE
// key as two separately quantized paths), shared by the append kernel and
// the fused append + decode.
//
// QuantMLA keeps a content path at INT4 or INT2 and a RoPE path at INT4
// ("QuantMLA: INT4 (and INT2) for both halves of the MLA cache", flowchart and
// Key findings).  Each channel group gets an asymmetric min/max scale and zero
// stored as fp16; codes come from the stored fp16 values with IEEE fp32
// subtract and divide and round-half-even, so that the result is
// bit-identical to a plain CPU implementation of the same definition (the
// library is built without fast-math or FP contraction for this reason).
#pragma once

#include "common.h"

namespace mla {

// Quantize the 8 values x[] held by this lane, as part of a group spread over
// LPG aligned lanes.  Returns the 8 codes packed at `bits` bits each (element
// e at bit e * bits) and the group's packed (S16 | Z16 << 16).
template <int BITS, int LPG>
__device__ __forceinline__ unsigned quant8(const float (&x)[8], unsigned& sz) {
  constexpr int kQmax = (1 << BITS) - 1;
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) { mn = fminf(mn, x[i]); mx = fmaxf(mx, x[i]); }
#pragma unroll
  for (int m = 1; m < LPG; m <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, m));
    mx = fmaxf(mx, __shfl_xor(mx, m));
  }
  // a -0 minimum or maximum is stored as +0 (min/max may return either zero)
  mn = mn + 0.0f;
  mx = mx + 0.0f;
  const float s32 = (mx - mn) / (float)kQmax;
  const _Float16 s16 = (_Float16)s32;   // round to nearest even
  const _Float16 z16 = (_Float16)mn;
  const float S = (float)s16, Z = (float)z16;
  unsigned packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    unsigned c = 0;
    if (S != 0.0f) {
      float t = (x[i] - Z) / S;          // IEEE fp32, correctly rounded
      float r = __builtin_rintf(t);      // ties to even
      r = fminf(fmaxf(r, 0.0f), (float)kQmax);
      c = (unsigned)r;
    }
    packed |= c << (i * BITS);
  }
  sz = (unsigned)__builtin_bit_cast(unsigned short, s16) |
       ((unsigned)__builtin_bit_cast(unsigned short, z16) << 16);
  return packed;
}

__device__ __forceinline__ void unpack8(const u32x4 w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { x[2 * i] = bf16_lo(w[i]); x[2 * i + 1] = bf16_hi(w[i]); }
}

// One wavefront (64 lanes) writes token `tok` of the page at `base` from the
// bf16 rows `lat` (512) and `rope` (64).  Lane l owns content channels
// [8l, 8l + 8); a group of G channels spans G / 8 neighbouring lanes, whose
// min/max are combined with xor-shuffles.  Lanes 0..7 also own the RoPE key
// (one group of 64).  The unquantized format copies the 1152-byte row.
template <int F>
__device__ __forceinline__ void append_row(const __bf16* __restrict__ lat, const __bf16* __restrict__ rope,
                                           uint8_t* __restrict__ base, int tok) {
  using Lay = PageLayout<F>;
  const int lane = threadIdx.x & 63;
  if constexpr (F == kBF16) {
    u32x4* row = (u32x4*)(base + (int64_t)tok * kD * 2);
    row[lane] = ((const u32x4*)lat)[lane];
    if (lane < 8) row[64 + lane] = ((const u32x4*)rope)[lane];
  } else {
    // content path: lane owns channels [8 lane, 8 lane + 8)
    {
      float x[8];
      unpack8(*(const u32x4*)(lat + 8 * lane), x);
      constexpr int kBits = Lay::kCBits, kG = Lay::kCGroup, kLpg = kG / 8;
      unsigned sz;
      const unsigned codes = quant8<kBits, kLpg>(x, sz);
      constexpr int kPerChunk = 128 / kBits;  // channels per 16-byte chunk
      const int ch = 8 * lane;
      const int chunk = ch / kPerChunk;
      const int byte = (ch % kPerChunk) * kBits / 8;
      uint8_t* cp = base + Lay::kCodesA + (chunk * kPage + tok) * 16 + byte;
      if (kBits == 4) *(unsigned*)cp = codes;
      else *(unsigned short*)cp = (unsigned short)codes;
      if ((lane % kLpg) == 0) {
        const int g = ch / kG;
        *(unsigned*)(base + Lay::kSzB + (g * kPage + tok) * 4) = sz;
      }
    }
    // RoPE path: INT4, one group of 64 over lanes 0..7 (other lanes mirror them)
    {
      const int rl = lane & 7;
      float x[8];
      unpack8(*(const u32x4*)(rope + 8 * rl), x);
      unsigned sz;
      const unsigned codes = quant8<4, 8>(x, sz);
      if (lane < 8) {
        const int ch = 8 * rl;
        *(unsigned*)(base + Lay::kCodesC + ((ch / 32) * kPage + tok) * 16 + (ch % 32) / 2) = codes;
        if (lane == 0) *(unsigned*)(base + Lay::kSzD + tok * 4) = sz;
      }
    }
  }
}

}  // namespace mla
