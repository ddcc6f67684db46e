// Stage 2 of the split scan fused with the per-head up-projection: the split
// partials of a row are merged by their log-sum-exp (KV-split reduction of the
// K3 time-share study, "Inside the blocks") and the merged latent row is
// multiplied by W_UV[h] (absorbed output side of the MLA operator-teardown
// page, section 4) in one pass, so the fp32 o_lat tile never leaves LDS.
//
// Workgroup = (head h, tile of R = 8 or 16 query rows t), 8 waves:
//   * merge: wave w merges rows t0 + w (and t0 + w + 8 when R = 16) as
//     combine_kernel does (split weights by readlane, the loads of up to 24
//     splits in flight (16 with 8-row tiles), empty splits never read) into an
//     fp32 tile in LDS; the split LSEs are read once.
//     Lane l owns
//     latent columns 4l..4l+3 and 256+4l..+3, so every load instruction covers
//     1 KiB of contiguous memory;
//   * W_UV[h] fragments (output rows 16w..16w+15, all 512 latent columns):
//     with 16-row tiles requested after the merge loads, so the merge waits
//     only on its own data and the weight loads overlap the LDS write and the
//     barrier; with 8-row tiles (few rows, latency-bound) requested first.
//     The workgroups of one head are 128 apart in the grid, hence on the same
//     XCD, and share W_UV[h] through its L2;
//   * up-projection: out^T[d, t] = sum_c W_UV[h][d][c] o_lat[t][c] on
//     v_mfma_f32_16x16x32_bf16 (16 rows d x 16 columns t, of which the tile's
//     R are real, x 32 latent columns c), the fp32 o_lat fed as a bf16 high
//     part plus a bf16 remainder (two MFMAs per step, ~16 significant bits).
// R = 8 keeps every merge concurrent and spreads few rows over more
// workgroups; R = 16 halves the W_UV reads per row where there are rows
// enough to fill the chip.
// In k-step ks, lane quad q holds latent columns 32ks + 8q .. +7 of both
// operands, so one instruction reads 64 contiguous bytes of each W_UV row.
#include "mla_device.hpp"
#include "decode.hpp"

namespace mla {

namespace {

constexpr int kTileCols = 16;     // MFMA columns: the tile's rows, then zero rows
constexpr int kSmallTileMaxRows = 32;  // T up to this: 8-row tiles, else 16-row tiles
constexpr int kOlatStride = kDc + 4;  // floats; the pad spreads the 16 rows of an MFMA read over the banks
constexpr int kMergeChunk = 24;       // splits whose loads are in flight together

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace

template <int kRows>
__global__ __launch_bounds__(512) void combine_up_kernel(const float* __restrict__ o_part,
                                                         const float* __restrict__ lse_part,
                                                         const __bf16* __restrict__ w_uv, int T, int num_splits,
                                                         __bf16* __restrict__ out, float* __restrict__ lse_out) {
  static_assert(kRows == 8 || kRows == 16, "one or two rows per wave");
  __shared__ __attribute__((aligned(16))) float olat[kTileCols * kOlatStride];
  const int h = blockIdx.x % kH;
  const int t0 = (blockIdx.x / kH) * kRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r = lane & 15;

  // W_UV[h] rows d = 16w + r, columns 32ks + 8q .. +7 for k-steps ks = 0..15.
  // With 8-row tiles (few rows: each load round is latency, not bandwidth)
  // they are requested first, so their latency overlaps the merge's; with
  // 16-row tiles after the merge loads, so the merge waits only on its own data.
  bf16x8 a[16];
  auto load_w = [&]() {
    const bf16x8* wp = reinterpret_cast<const bf16x8*>(w_uv + ((int64_t)h * kDhc + 16 * wave + r) * kDc + 8 * q);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) a[ks] = wp[4 * ks];
  };
  if constexpr (kRows == 8) load_w();

  // ---- merge rows t0 + w (+ 8) into LDS rows w (+ 8); zeros past the end,
  // never stored
  for (int rr = wave; rr < kTileCols; rr += 8) {
    f32x4v a0 = f32x4v{}, a1 = f32x4v{};
    const int tm = t0 + rr;
    if (rr < kRows && tm < T) {
      const int64_t row = (int64_t)tm * kH + h;
      const float* lp = lse_part + row * num_splits;
      const float* op = o_part + row * num_splits * kDc + 4 * lane;
      // up to 64 splits: one load round, lane s holding lse_s for the max, the
      // sum and the weights
      const float l0 = lane < num_splits ? lp[lane] : -INFINITY;
      float M = l0;
      for (int s = lane + 64; s < num_splits; s += 64) M = fmaxf(M, lp[s]);
      M = wave_max_f(M);
      float L = -INFINITY;
      if (M != -INFINITY) {
        float tot = expf(l0 - M);
        for (int s = lane + 64; s < num_splits; s += 64) tot += expf(lp[s] - M);
        L = M + logf(wave_sum_f(tot));
        // 8-row tiles hold W_UV's fragments during the merge: 16 splits in flight
        constexpr int kChunk = kRows == 8 ? 16 : kMergeChunk;
        f32x4v v0[kChunk], v1[kChunk];
        for (int b0 = 0; b0 < num_splits; b0 += 64) {  // blocks of 64 splits: lane k holds the weight of b0 + k
          const int b1 = min(num_splits, b0 + 64);
          const float lb = b0 == 0 ? l0 : (b0 + lane < num_splits ? lp[b0 + lane] : -INFINITY);
          const float wl = expf(lb - L);  // 0 when lse = -inf
          auto weight = [&](int s) {
            return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s - b0));
          };
          for (int s0 = b0; s0 < b1; s0 += kChunk) {
#pragma unroll
            for (int k = 0; k < kChunk; ++k) {
              if (s0 + k < b1 && weight(s0 + k) > 0.f) {
                v0[k] = *reinterpret_cast<const f32x4v*>(op + (int64_t)(s0 + k) * kDc);
                v1[k] = *reinterpret_cast<const f32x4v*>(op + (int64_t)(s0 + k) * kDc + kDc / 2);
              }
            }
#pragma unroll
            for (int k = 0; k < kChunk; ++k) {
              if (s0 + k < b1) {
                const float w = weight(s0 + k);
                if (w > 0.f) {
                  a0 += w * v0[k];
                  a1 += w * v1[k];
                }
              }
            }
          }
        }
      }
      if (lane == 0) lse_out[row] = L;
    }
    float* dst = olat + rr * kOlatStride + 4 * lane;
    *reinterpret_cast<f32x4v*>(dst) = a0;
    *reinterpret_cast<f32x4v*>(dst + kDc / 2) = a1;
  }

  if constexpr (kRows == 16) load_w();

  __syncthreads();

  // ---- up-projection of the tile: D[d][t], d = 16w + 4q + i, t = t0 + r
  f32x4 acc = f32x4{};
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const float* src = olat + r * kOlatStride + 32 * ks + 8 * q;
    const f32x4v x0 = *reinterpret_cast<const f32x4v*>(src);
    const f32x4v x1 = *reinterpret_cast<const f32x4v*>(src + 4);
    bf16x8 hi, lw;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = j < 4 ? x0[j] : x1[j - 4];
      hi[j] = (__bf16)v;
      lw[j] = (__bf16)(v - (float)hi[j]);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], lw, acc, 0, 0, 0);
  }
  const int t = t0 + r;
  if (r < kRows && t < T) {
    const bf16x4 o = {(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3]};
    *reinterpret_cast<bf16x4*>(out + ((int64_t)t * kH + h) * kDhc + 16 * wave + 4 * q) = o;
  }
}

hipError_t launch_combine_up(const float* o_part, const float* lse_part, const __bf16* w_uv, int T, int num_splits,
                             __bf16* out, float* lse, hipStream_t stream) {
  if (T <= kSmallTileMaxRows) {
    hipLaunchKernelGGL(combine_up_kernel<8>, dim3(kH * ((T + 7) / 8)), dim3(512), 0, stream, o_part, lse_part, w_uv,
                       T, num_splits, out, lse);
  } else {
    hipLaunchKernelGGL(combine_up_kernel<16>, dim3(kH * ((T + 15) / 16)), dim3(512), 0, stream, o_part, lse_part,
                       w_uv, T, num_splits, out, lse);
  }
  return hipGetLastError();
}

}  // namespace mla
