// The 4-bit latent cache: page layout and the row quantizer of the kernels
// that write it.
//
// The teardown page's NVFP4 gather (section 5) reads a 4-bit latent cache
// with 16-byte vector loads. gfx950's matrix cores take the OCP
// microscaling form of a 4-bit cache (MXFP4) directly, so this cache stores
// c_KV as E2M1 elements with one E8M0 scale per 32 consecutive dims of a
// token, and keeps k_R in bf16:
//   * block scale 2^k with k the smallest integer such that
//     max|block| <= 6 * 2^k, clamped to [-126, 127] (a zero block gets
//     2^-126), so no element saturates; stored as the byte k + 127;
//   * code = c / 2^k rounded to the nearest E2M1 value (0, 0.5, 1, 1.5, 2,
//     3, 4, 6), ties to the even code, with c's sign bit;
//   * two codes per byte, the even dim in the low nibble;
//   * stored value = E2M1 value of the code * 2^k.
// A page of 64 tokens holds three arrays, each 16-byte aligned:
//   [0, 16384)      64 rows x 256 code bytes (block u of a row = bytes 16u..16u+15)
//   [16384, 24576)  64 rows x 64 bf16 k_R
//   [24576, 25600)  64 rows x 16 scale bytes
#pragma once

#include "mla_device.hpp"

namespace mla {

constexpr int kMxBlock = 32;                                         // dims per scale
constexpr int kFp4RowBytes = kDc / 2;                                // 256
constexpr int kFp4RopeOffset = kPage * kFp4RowBytes;                 // 16384
constexpr int kFp4ScaleOffset = kFp4RopeOffset + kPage * kDr * 2;    // 24576
constexpr int kFp4PageBytes = kFp4ScaleOffset + kPage * (kDc / kMxBlock);  // 25600
static_assert(kFp4RopeOffset % 16 == 0 && kFp4ScaleOffset % 16 == 0 && kFp4PageBytes % 16 == 0,
              "every array of a 4-bit page starts on a 16-byte boundary");

// Scale exponent of a block whose largest magnitude is amax (finite, >= 0):
// amax = (1 + m / 2^23) * 2^(e - 127) fits 6 * 2^k = 1.5 * 2^(k + 2) exactly
// when k >= e - 129, plus one when the significand exceeds 1.5.
__device__ __forceinline__ int mx_scale_exponent(float amax) {
  const unsigned u = __float_as_uint(amax);
  int k = (int)(u >> 23) - 129 + ((u & 0x7FFFFFu) > 0x400000u ? 1 : 0);
  return k < -126 ? -126 : (k > 127 ? 127 : k);
}

// E2M1 code of x with |x| <= 6: the magnitude code counts the rounding
// boundaries at or below |x|; a boundary halfway between two values belongs
// to the one with the even code (0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0,
// 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4). neg is the sign bit to store.
__device__ __forceinline__ unsigned e2m1_code(float x, bool neg) {
  const float a = __builtin_fabsf(x);
  const unsigned m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return m | (neg ? 8u : 0u);
}

// One wave quantizes one 512-value row, 8 values per lane (lane l holds dims
// 8l..8l+7, so lanes 4u..4u+3 hold block u): returns the lane's 4 code bytes
// (byte j = dims 8l+2j (low nibble) and 8l+2j+1) and sets k to the scale
// exponent of the lane's block. x * 2^-k is exact down to the values far
// below the first rounding boundary.
__device__ __forceinline__ unsigned quantize_row_mxfp4(const bf16x8& x, int& k) {
  float v[8];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[j] = (float)x[j];
    amax = fmaxf(amax, __builtin_fabsf(v[j]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  k = mx_scale_exponent(amax);
  unsigned codes = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) codes |= e2m1_code(__builtin_ldexpf(v[j], -k), __builtin_signbit(v[j])) << (4 * j);
  return codes;
}

}  // namespace mla
