// Device-side types and paged-cache addressing shared by the MLA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

constexpr int kH = 128;
constexpr int kDhc = 128;
constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kRowElems = 576;
constexpr int kRowBytes = kRowElems * 2;      // 1152
constexpr int kPage = 64;
constexpr int kPageBytes = kPage * kRowBytes;  // 73728

// Tokens of sequence b that the cache can hold: L clamped to [0, max_pages*64].
__device__ __forceinline__ int clamp_len(int L, int max_pages) {
  const int cap = max_pages * kPage;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// Physical page of logical page p of sequence b, clamped into the cache so
// that a bad table entry can never address memory outside it.
__device__ __forceinline__ int64_t physical_page(const int32_t* __restrict__ block_table, int max_pages,
                                                 int b, int p, int64_t num_pages) {
  int64_t id = block_table[(int64_t)b * max_pages + p];
  if (id < 0) id = 0;
  if (id >= num_pages) id = num_pages - 1;
  return id;
}

// Byte address of token t (logical) of sequence b in the paged cache.
__device__ __forceinline__ const char* token_row(const char* __restrict__ kv, const int32_t* __restrict__ block_table,
                                                 int max_pages, int b, int t, int64_t num_pages) {
  const int64_t page = physical_page(block_table, max_pages, b, t >> 6, num_pages);
  return kv + page * kPageBytes + (int64_t)(t & (kPage - 1)) * kRowBytes;
}

// The lane id, recomputed where it is used: volatile asm, so the compiler
// neither merges it with another lane-id computation (which would keep that
// value live from one phase of a kernel into a much later one) nor hoists it.
__device__ __forceinline__ int lane_opaque() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Max and sum of a float over the 64 lanes, returned to every lane: an
// inclusive scan on DPP (shifts by 1, 2, 4 and 8 inside each 16-lane row, then
// lane 15's value into rows 1 and 3 and lane 31's into rows 2 and 3), read at
// lane 63. Lanes shifted in read the identity (-inf, resp. 0). Six dependent
// VALU steps with a fixed order, where a __shfl ladder waits on six
// ds_bpermute round trips.
template <bool kMax>
__device__ __forceinline__ float wave_reduce_dpp(float v) {
  const int id = kMax ? __builtin_bit_cast(int, -INFINITY) : 0;
  auto step = [&](int u) {
    const float f = __builtin_bit_cast(float, u);
    v = kMax ? fmaxf(v, f) : v + f;
  };
  step(__builtin_amdgcn_update_dpp(id, __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, false));  // row_shr:1
  step(__builtin_amdgcn_update_dpp(id, __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, false));  // row_shr:2
  step(__builtin_amdgcn_update_dpp(id, __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, false));  // row_shr:4
  step(__builtin_amdgcn_update_dpp(id, __builtin_bit_cast(int, v), 0x118, 0xf, 0xf, false));  // row_shr:8
  step(__builtin_amdgcn_update_dpp(id, __builtin_bit_cast(int, v), 0x142, 0xa, 0xf, false));  // row_bcast:15
  step(__builtin_amdgcn_update_dpp(id, __builtin_bit_cast(int, v), 0x143, 0xc, 0xf, false));  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_max_dpp(float v) { return wave_reduce_dpp<true>(v); }
__device__ __forceinline__ float wave_sum_dpp(float v) { return wave_reduce_dpp<false>(v); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] = 7, lgkmcnt [11:8] = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace mla
