// The 8-bit latent cache: page layout and the row quantizer of the kernels
// that write it.
//
// The MLA operator-teardown page gathers a quantized (4-bit) latent cache
// with 16-byte vector loads that need a 16-byte aligned page base and
// dimension offset (section 5) but fixes no format for this hardware. This
// cache stores c_KV in OCP FP8 E4M3 (the 8-bit float gfx950 converts in one
// instruction) with one power-of-two scale per token, and keeps k_R in bf16:
//   * scale 2^k with k the smallest integer such that max|c_KV| <= 448 * 2^k,
//     clamped to [-126, 127] (an all-zero row gets 2^-126), so no element of
//     the row saturates;
//   * code = c / 2^k rounded to nearest, ties to even, with c's sign bit;
//   * stored value = E4M3 value of the code * 2^k.
// A page of 64 tokens holds three arrays, each 16-byte aligned:
//   [0, 32768)      64 rows x 512 codes
//   [32768, 40960)  64 rows x 64 bf16 k_R
//   [40960, 41216)  64 float32 scales (always exactly 2^k)
#pragma once

#include "mla_device.hpp"

namespace mla {

constexpr int kFp8RopeOffset = kPage * kDc;                     // 32768
constexpr int kFp8ScaleOffset = kFp8RopeOffset + kPage * kDr * 2;  // 40960
constexpr int kFp8PageBytes = kFp8ScaleOffset + kPage * 4;        // 41216
static_assert(kFp8RopeOffset % 16 == 0 && kFp8ScaleOffset % 16 == 0 && kFp8PageBytes % 16 == 0,
              "every array of an 8-bit page starts on a 16-byte boundary");

// Scale exponent of a row whose largest magnitude is amax (finite, >= 0):
// amax = (1 + m / 2^23) * 2^(e - 127) fits 448 * 2^k = 1.75 * 2^(k + 8) exactly
// when k >= e - 135, plus one when the significand exceeds 1.75.
__device__ __forceinline__ int fp8_scale_exponent(float amax) {
  const unsigned u = __float_as_uint(amax);
  int k = (int)(u >> 23) - 135 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return k < -126 ? -126 : (k > 127 ? 127 : k);
}

// One wave quantizes one 512-value row, 8 values per lane (lane l holds
// values 8l..8l+7): returns the lane's 8 codes (byte j = value 8l+j) and sets
// k to the row's scale exponent (the same in every lane). x * 2^-k is exact
// (a bf16 value times a power of two, at most 448 in magnitude), and
// v_cvt_pk_fp8_f32 rounds it to nearest even.
__device__ __forceinline__ uint2 quantize_row_fp8(const bf16x8& x, int& k) {
  float v[8];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[j] = (float)x[j];
    amax = fmaxf(amax, __builtin_fabsf(v[j]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  k = fp8_scale_exponent(amax);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = __builtin_ldexpf(v[j], -k);
  int d0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  d0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], d0, true);
  int d1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
  d1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], d1, true);
  return make_uint2((unsigned)d0, (unsigned)d1);
}

__device__ __forceinline__ float fp8_scale_value(int k) { return __uint_as_float((unsigned)(k + 127) << 23); }

}  // namespace mla
