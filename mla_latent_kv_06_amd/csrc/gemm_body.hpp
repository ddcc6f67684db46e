// Per-head projections around the absorbed decode, on bf16 matrix cores
// (workgroup bodies; gemm.hip launches them as kernels, step.hip as phases).
//
// absorb:   q_abs[t, h, c] = sum_d q_c[t, h, d] W_UK[h, d, c]   (d: 128, c: 512)
//           (absorbed path of the MLA operator-teardown page, section 4)
// up-proj:  out[t, h, d]   = sum_c o_lat[t, h, c] W_UV[h, d, c]  (c: 512, d: 128)
//
// Both are computed transposed, D^T = W^T-ish . X^T, so that each lane of the
// 32x32 accumulator owns one token and 4-runs of consecutive output columns.
// At decode sizes both are bound by reading the 16 MiB weight once.
#pragma once

#include "mla_device.hpp"
#include "decode.hpp"

namespace mla {

namespace {

constexpr int kAbsCols = 128;               // output columns c per workgroup (4 waves x 32)
constexpr int kAbsLdsStride = kAbsCols * 2 + 16;  // padded W row in LDS (bytes)

}  // namespace

constexpr int kAbsorbLdsBytes = kDhc * kAbsLdsStride;
constexpr int kUpProjLdsBytes = 4 * 4 * 64 * 16;
constexpr int kAbsorbItems = kH * (kDc / kAbsCols);  // 512
constexpr int kAbsorbTokens = 512;  // tokens per absorb workgroup: longer chunks spread over more workgroups
                                    // (1024 tokens: 44 us, against 53 us with 128 and 47 us with 256)
constexpr int kUpProjItems = kH * 4;                 // 512

// Workgroup = (head h, 128-column block cb, tokens [t_begin, t_end)).
// W_UK[h][:, cb*128 .. +128] is staged in LDS once; the A operand (W^T: 32
// columns c x 16 dims d per lane group) is then read with transposed LDS reads
// and kept in registers for the workgroup's token tiles. The LDS then stages
// each 32-token tile both ways: the queries arrive as whole 256-byte rows
// (q_c[t][h], 16 lanes per row) and are read back in the MFMA's layout, and the
// 32 x 128 output tile is written to LDS and stored as whole 256-byte rows of
// q_abs. Loaded or stored straight in the MFMA layout, every instruction would
// touch 32 token rows 32 KB (q_c) or 128 KB (q_abs) apart in 16-32 byte pieces;
// staged, the 1024-token absorb takes 54 us instead of 96.
// item = (head, column block) = h * 4 + cb; lds: kAbsorbLdsBytes, 16-byte aligned
__device__ __forceinline__ void absorb_body(char* __restrict__ lds, int item, const __bf16* __restrict__ q_c,
                                            const __bf16* __restrict__ w_uk, __bf16* __restrict__ q_abs, int t_begin,
                                            int t_end) {
  const int h = item >> 2;
  const int cb = item & 3;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, lo = lane & 31;

  // B operand (q_c^T: dims d = 16ks + 8g + 0..7 of token t0 + lo) of a token
  // tile: loaded as whole rows (thread tid: 16-byte chunks tid and tid + 256
  // of the tile, i.e. token chunk >> 4, bytes 16 (chunk & 15)), staged in LDS,
  // read back per lane; the first tile is requested before the weights so
  // both latencies overlap
  bf16x8 bq[8];
  f32x4 qraw[2];
  auto load_q = [&](int t0) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = k * 256 + tid, t = t0 + (c >> 4);
      qraw[k] = t < t_end ? *reinterpret_cast<const f32x4*>(q_c + ((int64_t)t * kH + h) * kDhc + (c & 15) * 8) : f32x4{};
    }
  };
  char* const qst = lds + 32 * kAbsLdsStride;  // query tile: 32 rows of 256 bytes (+16 padding)
  auto stage_q = [&]() {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = k * 256 + tid;
      *reinterpret_cast<f32x4*>(qst + (c >> 4) * kAbsLdsStride + (c & 15) * 16) = qraw[k];
    }
  };
  auto read_q = [&]() {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) bq[ks] = *reinterpret_cast<const bf16x8*>(qst + lo * kAbsLdsStride + (2 * ks + g) * 16);
  };
  load_q(t_begin);

  // stage W rows d = 0..127, columns cb*128 .. +128 (256 bytes per row)
  const char* wsrc = reinterpret_cast<const char*>(w_uk + ((int64_t)h * kDhc) * kDc + cb * kAbsCols);
  f32x4 wv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int q = k * 256 + tid;        // 16-byte chunk: row q/16, chunk q%16
    wv[k] = *reinterpret_cast<const f32x4*>(wsrc + (int64_t)(q >> 4) * kDc * 2 + (q & 15) * 16);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int q = k * 256 + tid;
    *reinterpret_cast<f32x4*>(lds + (q >> 4) * kAbsLdsStride + (q & 15) * 16) = wv[k];
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

  __syncthreads();  // every wave has its A fragments: the LDS now stages query and output tiles
  for (int t0 = t_begin; t0 < t_end; t0 += 32) {
    if (t0 > t_begin) __syncthreads();  // the previous tile has been read and stored
    stage_q();
    __syncthreads();
    read_q();
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], bq[ks], acc, 0, 0, 0);
    if (t0 + 32 < t_end) load_q(t0 + 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x4 o = {(__bf16)acc[4 * q], (__bf16)acc[4 * q + 1], (__bf16)acc[4 * q + 2], (__bf16)acc[4 * q + 3]};
      *reinterpret_cast<bf16x4*>(lds + lo * kAbsLdsStride + (wave * 32 + 8 * q + 4 * g) * 2) = o;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = k * 256 + tid, row = c >> 4, ch = c & 15;
      if (t0 + row < t_end)
        *reinterpret_cast<f32x4*>(q_abs + ((int64_t)(t0 + row) * kH + h) * kDc + cb * kAbsCols + ch * 8) =
            *reinterpret_cast<const f32x4*>(lds + row * kAbsLdsStride + ch * 16);
    }
  }
}

// Workgroup = (head h, block of 32 rows d), split-K over its 4 waves: wave w
// covers latent columns c in [128w, 128w + 128) and all 32 rows, then the
// four partial tiles are added in LDS in a fixed order. Within a k-step, lane
// group g holds c = 128w + 64g + 8ks + 0..7 for both operands (any common
// permutation of the reduction index gives the same sum), so every lane reads
// 128 contiguous bytes of W_UV and 256 of o_lat, all issued up front.
// A = W_UV[h][d][c] rows; B = o_lat^T split into a bf16 high part and a bf16
// remainder (two MFMAs per step).
// x: the workgroup's place in a grid of 512 (its XCD is x & 7); red: LDS of
// kUpProjLdsBytes, 16-byte aligned
__device__ __forceinline__ void up_proj_body(f32x4 (*__restrict__ red)[4][64], int x, const float* __restrict__ o_lat,
                                             const __bf16* __restrict__ w_uv, __bf16* __restrict__ out, int T,
                                             int wg_per_xcd) {
  // x -> (h, row block) with the 4 row blocks of a head on one XCD, so they
  // share its o_lat rows in L2
  const int id = (x & 7) * wg_per_xcd + (x >> 3);
  if (id >= kH * 4) return;
  const int h = id >> 2;
  const int db = id & 3;
  const int lane = lane_opaque();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, lo = lane & 31;
  const int kc = 128 * wave + 64 * g;  // first latent column of this lane's slice

  const bf16x8* wp = reinterpret_cast<const bf16x8*>(w_uv + ((int64_t)h * kDhc + db * 32 + lo) * kDc + kc);
  bf16x8 a[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) a[ks] = wp[ks];

  for (int t0 = 0; t0 < T; t0 += 32) {
    const int t = t0 + lo;
    const bool tv = t < T;
    const f32x4* xp = reinterpret_cast<const f32x4*>(o_lat + ((int64_t)(tv ? t : 0) * kH + h) * kDc + kc);
    f32x4 xv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) xv[k] = tv ? xp[k] : f32x4{};
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8 hi, lw;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = xv[2 * ks + (j >> 2)][j & 3];
        hi[j] = (__bf16)v;
        lw[j] = (__bf16)(v - (float)hi[j]);
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], hi, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], lw, acc, 0, 0, 0);
    }
    if (t0 > 0) __syncthreads();  // the previous tile's sums have been read
#pragma unroll
    for (int q = 0; q < 4; ++q) red[wave][q][lane] = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    __syncthreads();
    // wave w finishes register quad w: rows d = 32db + 8w + 4g + 0..3 of token t
    const f32x4 r = ((red[0][wave][lane] + red[1][wave][lane]) + red[2][wave][lane]) + red[3][wave][lane];
    if (tv) {
      const bf16x4 o = {(__bf16)r[0], (__bf16)r[1], (__bf16)r[2], (__bf16)r[3]};
      *reinterpret_cast<bf16x4*>(out + ((int64_t)t * kH + h) * kDhc + db * 32 + 8 * wave + 4 * g) = o;
    }
  }
}

}  // namespace mla
