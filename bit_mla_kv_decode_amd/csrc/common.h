// Shared device-side definitions of the gfx950 low-bit MLA cache library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Cache shape: absorbed MLA keeps a 512-d content latent and a 64-d RoPE key
// per token, in pages of 64 tokens.
constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kD = kDc + kDr;
constexpr int kPage = 64;

enum Format : int { kC4R4 = 0, kC2R4 = 1, kBF16 = 2 };

// Byte offsets of the page regions (layout documented in mla_lowbit.h).
template <int F> struct PageLayout;
template <> struct PageLayout<kC4R4> {
  static constexpr int kCBits = 4, kCGroup = 64;
  static constexpr int kCodesA = 0;                       // 16 chunks x 64 tokens x 16 B
  static constexpr int kSzB = 16 * kPage * 16;             // 8 groups x 64 tokens x 4 B
  static constexpr int kCodesC = kSzB + 8 * kPage * 4;     // 2 chunks x 64 x 16 B
  static constexpr int kSzD = kCodesC + 2 * kPage * 16;    // 1 group x 64 x 4 B
  static constexpr int kBytes = kSzD + kPage * 4;          // 20736
};
template <> struct PageLayout<kC2R4> {
  static constexpr int kCBits = 2, kCGroup = 32;
  static constexpr int kCodesA = 0;                       // 8 chunks x 64 x 16 B
  static constexpr int kSzB = 8 * kPage * 16;              // 16 groups x 64 x 4 B
  static constexpr int kCodesC = kSzB + 16 * kPage * 4;
  static constexpr int kSzD = kCodesC + 2 * kPage * 16;
  static constexpr int kBytes = kSzD + kPage * 4;          // 14592
};
template <> struct PageLayout<kBF16> {
  static constexpr int kBytes = kPage * kD * 2;            // 73728
};
static_assert(PageLayout<kC4R4>::kBytes == 20736, "C4R4 page size");
static_assert(PageLayout<kC2R4>::kBytes == 14592, "C2R4 page size");

__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

__device__ __forceinline__ float half_bits_to_f32(unsigned h) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xFFFFu));
}

// Two fp32 values to a packed pair of bf16 (round to nearest even), first in the low half.
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(unsigned, v);
}

}  // namespace mla
