// Per-head projections around the absorbed decode, on bf16 matrix cores.
//
// absorb:   q_abs[t, h, c] = sum_d q_c[t, h, d] W_UK[h, d, c]   (d: 128, c: 512)
//           (absorbed path of the MLA operator-teardown page, section 4)
// up-proj:  out[t, h, d]   = sum_c o_lat[t, h, c] W_UV[h, d, c]  (c: 512, d: 128)
//
// Both are computed transposed, D^T = W^T-ish . X^T, so that each lane of the
// 32x32 accumulator owns one token and 4-runs of consecutive output columns,
// which become 8-byte bf16 stores. At decode sizes both are bound by reading
// the 16 MiB weight once.
#include "mla_device.hpp"
#include "decode.hpp"

namespace mla {

namespace {

constexpr int kAbsCols = 128;               // output columns c per workgroup (4 waves x 32)
constexpr int kAbsLdsStride = kAbsCols * 2 + 16;  // padded W row in LDS (bytes)

}  // namespace

// Workgroup = (head h, 128-column block cb). W_UK[h][:, cb*128 .. +128] is
// staged in LDS once; the A operand (W^T: 32 columns c x 16 dims d per lane
// group) is then read with transposed LDS reads and kept in registers for all
// token tiles.
__global__ __launch_bounds__(256) void absorb_kernel(const __bf16* __restrict__ q_c, const __bf16* __restrict__ w_uk,
                                                     __bf16* __restrict__ q_abs, int T) {
  __shared__ __attribute__((aligned(16))) char lds[kDhc * kAbsLdsStride];
  const int h = blockIdx.x >> 2;
  const int cb = blockIdx.x & 3;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lo = lane & 31;

  // stage W rows d = 0..127, columns cb*128 .. +128 (256 bytes per row)
  const char* wsrc = reinterpret_cast<const char*>(w_uk + ((int64_t)h * kDhc) * kDc + cb * kAbsCols);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int q = k * 256 + tid;        // 16-byte chunk: row q/16, chunk q%16
    const int d = q >> 4, ch = q & 15;
    const f32x4 v = *reinterpret_cast<const f32x4*>(wsrc + (int64_t)d * kDc * 2 + ch * 16);
    *reinterpret_cast<f32x4*>(lds + d * kAbsLdsStride + ch * 16) = v;
  }
  __syncthreads();

  // A fragments for the wave's 32 columns, k-steps ks = 0..7 (d = 16ks + 8g + j)
  bf16x8 af[8];
  {
    const int G = lane >> 4, ii = lane & 15;
    const int col = wave * 32 + 16 * (G & 1) + 4 * (ii & 3);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      // lane group g holds k = 8g..8g+7: rows d = 16ks + 8g + 0..3, then + 4..7
      const int d0 = 16 * ks + 8 * (G >> 1) + (ii >> 2);
      const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lds + d0 * kAbsLdsStride + col * 2));
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lds + (d0 + 4) * kAbsLdsStride + col * 2));
      const bf16x4 b0 = __builtin_bit_cast(bf16x4, v0);
      const bf16x4 b1 = __builtin_bit_cast(bf16x4, v1);
      af[ks] = bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    }
  }

  const int c0 = cb * kAbsCols + wave * 32;
  for (int t0 = 0; t0 < T; t0 += 32) {
    const int t = t0 + lo;
    const bool tv = t < T;
    const bf16x8* qrow = reinterpret_cast<const bf16x8*>(q_c + ((int64_t)(tv ? t : 0) * kH + h) * kDhc);
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 bq = tv ? qrow[2 * ks + g] : bf16x8{};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], bq, acc, 0, 0, 0);
    }
    if (tv) {
      __bf16* orow = q_abs + ((int64_t)t * kH + h) * kDc + c0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x4 o = {(__bf16)acc[4 * q], (__bf16)acc[4 * q + 1], (__bf16)acc[4 * q + 2], (__bf16)acc[4 * q + 3]};
        *reinterpret_cast<bf16x4*>(orow + 8 * q + 4 * g) = o;
      }
    }
  }
}

// Workgroup = (head h, 64-row half of d), 2 waves of 32 rows d each, looping
// over token tiles. A = W_UV[h][d][c] rows (contiguous 16-byte reads);
// B = o_lat^T split into bf16 high part and bf16 remainder (two MFMAs per step).
__global__ __launch_bounds__(128) void up_proj_kernel(const float* __restrict__ o_lat, const __bf16* __restrict__ w_uv,
                                                      __bf16* __restrict__ out, int T) {
  const int h = blockIdx.x >> 1;
  const int half = blockIdx.x & 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lo = lane & 31;
  const int d0 = half * 64 + wave * 32;

  const bf16x8* wrow = reinterpret_cast<const bf16x8*>(w_uv + ((int64_t)h * kDhc + d0 + lo) * kDc);
  for (int t0 = 0; t0 < T; t0 += 32) {
    const int t = t0 + lo;
    const bool tv = t < T;
    const float* orow = o_lat + ((int64_t)(tv ? t : 0) * kH + h) * kDc;
    f32x16 acc = f32x16{};
#pragma unroll 4
    for (int ks = 0; ks < 32; ++ks) {
      const bf16x8 a = wrow[2 * ks + g];
      f32x4 x0 = f32x4{}, x1 = f32x4{};
      if (tv) {
        x0 = *reinterpret_cast<const f32x4*>(orow + 16 * ks + 8 * g);
        x1 = *reinterpret_cast<const f32x4*>(orow + 16 * ks + 8 * g + 4);
      }
      bf16x8 hi, lw;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hi[j] = (__bf16)x0[j];
        hi[4 + j] = (__bf16)x1[j];
        lw[j] = (__bf16)(x0[j] - (float)hi[j]);
        lw[4 + j] = (__bf16)(x1[j] - (float)hi[4 + j]);
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, hi, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, lw, acc, 0, 0, 0);
    }
    if (tv) {
      __bf16* op = out + ((int64_t)t * kH + h) * kDhc + d0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x4 o = {(__bf16)acc[4 * q], (__bf16)acc[4 * q + 1], (__bf16)acc[4 * q + 2], (__bf16)acc[4 * q + 3]};
        *reinterpret_cast<bf16x4*>(op + 8 * q + 4 * g) = o;
      }
    }
  }
}

hipError_t launch_absorb(const __bf16* q_c, const __bf16* w_uk, __bf16* q_abs, int T, hipStream_t stream) {
  hipLaunchKernelGGL(absorb_kernel, dim3(kH * (kDc / kAbsCols)), dim3(256), 0, stream, q_c, w_uk, q_abs, T);
  return hipGetLastError();
}

hipError_t launch_up_proj(const float* o_lat, const __bf16* w_uv, __bf16* out, int T, hipStream_t stream) {
  hipLaunchKernelGGL(up_proj_kernel, dim3(kH * 2), dim3(128), 0, stream, o_lat, w_uv, out, T);
  return hipGetLastError();
}

}  // namespace mla
