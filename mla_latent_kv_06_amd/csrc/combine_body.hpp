// Stage 2 of absorbed MLA decode: merge the split partials of each
// (sequence, query, head) row by their log-sum-exp (KV-split reduction of the
// K3 time-share study, "Inside the blocks").
//
// One wave per row: lane k holds the LSE of split k (of each block of 64),
// max and sum come from DPP wave reductions, and each split's weight is
// broadcast with readlane. Lane l owns latent columns 4l..4l+3 and
// 256+4l..+3, so each load instruction covers 1 KiB of contiguous memory; up
// to 16 splits' loads are in flight. Splits with LSE = -inf
// are empty; their partial rows were never written and are not read.
#pragma once

#include "mla_device.hpp"
#include "decode.hpp"

namespace mla {

constexpr int kCombineChunk = 16;  // splits whose loads are in flight together

// item: a block of 4 rows, one per wave
__device__ __forceinline__ void combine_body(int item, const float* __restrict__ o_part,
                                             const float* __restrict__ lse_part, int rows, int num_splits,
                                             float* __restrict__ o_lat, float* __restrict__ lse) {
  const int lane = lane_opaque();
  const int row = __builtin_amdgcn_readfirstlane(item * 4 + (threadIdx.x >> 6));
  if (row >= rows) return;
  const float* lp = lse_part + (int64_t)row * num_splits;
  const float* op = o_part + (int64_t)row * num_splits * kDc + 4 * lane;
  float* orow = o_lat + (int64_t)row * kDc + 4 * lane;

  float M = -INFINITY;
  for (int s = lane; s < num_splits; s += 64) M = fmaxf(M, lp[s]);
  M = wave_max_dpp(M);
  if (M == -INFINITY) {  // every split empty
    *reinterpret_cast<f32x4*>(orow) = f32x4{};
    *reinterpret_cast<f32x4*>(orow + kDc / 2) = f32x4{};
    if (lane == 0) lse[row] = -INFINITY;
    return;
  }
  float tot = 0.f;
  for (int s = lane; s < num_splits; s += 64) tot += expf(lp[s] - M);
  tot = wave_sum_dpp(tot);
  const float L = M + logf(tot);

  f32x4 a0 = f32x4{}, a1 = f32x4{};
  f32x4 v0[kCombineChunk], v1[kCombineChunk];
  float wl = 0.f;  // lane k: weight of split (s0 & ~63) + k
  auto weight = [&](int s) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s & 63));
  };
  for (int s0 = 0; s0 < num_splits; s0 += kCombineChunk) {
    if ((s0 & 63) == 0) wl = s0 + lane < num_splits ? expf(lp[s0 + lane] - L) : 0.f;  // 0 when lse = -inf
#pragma unroll
    for (int k = 0; k < kCombineChunk; ++k) {
      if (s0 + k < num_splits && weight(s0 + k) > 0.f) {
        v0[k] = *reinterpret_cast<const f32x4*>(op + (int64_t)(s0 + k) * kDc);
        v1[k] = *reinterpret_cast<const f32x4*>(op + (int64_t)(s0 + k) * kDc + kDc / 2);
      }
    }
#pragma unroll
    for (int k = 0; k < kCombineChunk; ++k) {
      if (s0 + k < num_splits) {
        const float w = weight(s0 + k);
        if (w > 0.f) {
          a0 += w * v0[k];
          a1 += w * v1[k];
        }
      }
    }
  }
  *reinterpret_cast<f32x4*>(orow) = a0;
  *reinterpret_cast<f32x4*>(orow + kDc / 2) = a1;
  if (lane == 0) lse[row] = L;
}

}  // namespace mla
