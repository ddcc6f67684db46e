// The step before the decode path: write a chunk of new tokens into the paged
// latent cache and rotate the decoupled RoPE parts of keys and queries.
//
// RoPE is applied in fp32 from an fp32 table (the precision the MLA
// operator-teardown page prescribes: the plugin's RoPE compute type is fp32,
// section 3, and a table generated in fp32 with fp32 multiply-adds cures the
// phase error of an fp16 rotation, section 4). Pair j of a 64-value vector is
// (x[2j], x[2j+1]) and turns by p * theta_j at position p; the table holds
// cos and sin of that angle for every (p, j), built on the host in double.
// Token i of an s_q-token chunk of sequence b has position L_b - s_q + i,
// L_b counting the chunk.
#include <cmath>

#include "mla_device.hpp"
#include "append.hpp"
#include "fp8_cache.hpp"
#include "mxfp4_cache.hpp"

namespace mla {

namespace {

// Position of chunk token i of sequence b, or -1 if it is negative or not
// below cap (the rotation table's length, and for the cache also the block
// table's capacity).
__device__ __forceinline__ int chunk_position(const int32_t* __restrict__ seqlens, int b, int i, int s_q,
                                              int64_t cap) {
  const int64_t p = (int64_t)seqlens[b] - s_q + i;
  return (p < 0 || p >= cap) ? -1 : (int)p;
}

// (x0, x1) turned by the angle whose cos/sin are cs, in fp32, then rounded
// once to bf16 (round to nearest even)
__device__ __forceinline__ bf16x2 rotate_pair(bf16x2 x, float2 cs) {
  const float x0 = (float)x[0], x1 = (float)x[1];
  const float y0 = __builtin_fmaf(x0, cs.x, -x1 * cs.y);
  const float y1 = __builtin_fmaf(x0, cs.y, x1 * cs.x);
  return bf16x2{(__bf16)y0, (__bf16)y1};
}

}  // namespace

// One wave per chunk token: 64 lanes copy the 1024-byte c_KV part in one
// 16-byte store each; lanes 0..31 rotate one k_R pair each.
__global__ __launch_bounds__(256) void append_latent_kernel(const __bf16* __restrict__ c_new,
                                                            const __bf16* __restrict__ kr_new,
                                                            const float2* __restrict__ rope, int max_pos,
                                                            char* __restrict__ kv, int64_t num_pages,
                                                            const int32_t* __restrict__ block_table, int max_pages,
                                                            const int32_t* __restrict__ seqlens, int T, int s_q) {
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const int b = t / s_q, i = t - b * s_q;
  const int64_t cap = (int64_t)max_pages * kPage < max_pos ? (int64_t)max_pages * kPage : max_pos;
  const int p = chunk_position(seqlens, b, i, s_q, cap);
  if (p < 0) return;
  const int64_t page = physical_page(block_table, max_pages, b, p >> 6, num_pages);
  char* row = kv + page * kPageBytes + (int64_t)(p & (kPage - 1)) * kRowBytes;
  const f32x4 c = reinterpret_cast<const f32x4*>(c_new + (int64_t)t * kDc)[lane];
  reinterpret_cast<f32x4*>(row)[lane] = c;
  if (lane < kDr / 2) {
    const bf16x2 x = reinterpret_cast<const bf16x2*>(kr_new + (int64_t)t * kDr)[lane];
    const float2 cs = rope[(int64_t)p * (kDr / 2) + lane];
    reinterpret_cast<bf16x2*>(row + kDc * 2)[lane] = rotate_pair(x, cs);
  }
}

// The same append into the 8-bit cache: one wave per chunk token quantizes
// its c_KV row (8 values per lane, 8 code bytes stored per lane), lanes
// 0..31 rotate one k_R pair each, lane 0 stores the token's scale.
__global__ __launch_bounds__(256) void append_latent_fp8_kernel(const __bf16* __restrict__ c_new,
                                                                const __bf16* __restrict__ kr_new,
                                                                const float2* __restrict__ rope, int max_pos,
                                                                char* __restrict__ kv, int64_t num_pages,
                                                                const int32_t* __restrict__ block_table,
                                                                int max_pages, const int32_t* __restrict__ seqlens,
                                                                int T, int s_q) {
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const int b = t / s_q, i = t - b * s_q;
  const int64_t cap = (int64_t)max_pages * kPage < max_pos ? (int64_t)max_pages * kPage : max_pos;
  const int p = chunk_position(seqlens, b, i, s_q, cap);
  if (p < 0) return;
  const int64_t page = physical_page(block_table, max_pages, b, p >> 6, num_pages);
  char* base = kv + page * kFp8PageBytes;
  const int r = p & (kPage - 1);
  int k;
  const uint2 codes = quantize_row_fp8(reinterpret_cast<const bf16x8*>(c_new + (int64_t)t * kDc)[lane], k);
  reinterpret_cast<uint2*>(base + r * kDc)[lane] = codes;
  if (lane < kDr / 2) {
    const bf16x2 x = reinterpret_cast<const bf16x2*>(kr_new + (int64_t)t * kDr)[lane];
    const float2 cs = rope[(int64_t)p * (kDr / 2) + lane];
    reinterpret_cast<bf16x2*>(base + kFp8RopeOffset + r * kDr * 2)[lane] = rotate_pair(x, cs);
  }
  if (lane == 0) reinterpret_cast<float*>(base + kFp8ScaleOffset)[r] = fp8_scale_value(k);
}

// bf16 pages [num_pages, 64, 576] -> 8-bit pages [num_pages, 41216 bytes],
// page for page: one wave per token row.
__global__ __launch_bounds__(256) void quantize_cache_fp8_kernel(const char* __restrict__ kv, int64_t num_pages,
                                                                 char* __restrict__ out) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= num_pages * kPage) return;
  const int64_t page = row >> 6;
  const int r = (int)(row & (kPage - 1));
  const char* src = kv + page * kPageBytes + (int64_t)r * kRowBytes;
  char* base = out + page * kFp8PageBytes;
  int k;
  const uint2 codes = quantize_row_fp8(reinterpret_cast<const bf16x8*>(src)[lane], k);
  reinterpret_cast<uint2*>(base + r * kDc)[lane] = codes;
  if (lane < kDr * 2 / 16)
    reinterpret_cast<f32x4*>(base + kFp8RopeOffset + r * kDr * 2)[lane] =
        reinterpret_cast<const f32x4*>(src + kDc * 2)[lane];
  if (lane == 0) reinterpret_cast<float*>(base + kFp8ScaleOffset)[r] = fp8_scale_value(k);
}

// The append into the 4-bit cache: one wave per chunk token, c_KV quantized
// per 32-dim block, k_R rotated as in the bf16 cache.
__global__ __launch_bounds__(256) void append_latent_mxfp4_kernel(const __bf16* __restrict__ c_new,
                                                                  const __bf16* __restrict__ kr_new,
                                                                  const float2* __restrict__ rope, int max_pos,
                                                                  char* __restrict__ kv, int64_t num_pages,
                                                                  const int32_t* __restrict__ block_table,
                                                                  int max_pages, const int32_t* __restrict__ seqlens,
                                                                  int T, int s_q) {
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const int b = t / s_q, i = t - b * s_q;
  const int64_t cap = (int64_t)max_pages * kPage < max_pos ? (int64_t)max_pages * kPage : max_pos;
  const int p = chunk_position(seqlens, b, i, s_q, cap);
  if (p < 0) return;
  const int64_t page = physical_page(block_table, max_pages, b, p >> 6, num_pages);
  char* base = kv + page * kFp4PageBytes;
  const int r = p & (kPage - 1);
  int k;
  const unsigned codes = quantize_row_mxfp4(reinterpret_cast<const bf16x8*>(c_new + (int64_t)t * kDc)[lane], k);
  reinterpret_cast<unsigned*>(base + r * kFp4RowBytes)[lane] = codes;
  if (lane < kDr / 2) {
    const bf16x2 x = reinterpret_cast<const bf16x2*>(kr_new + (int64_t)t * kDr)[lane];
    const float2 cs = rope[(int64_t)p * (kDr / 2) + lane];
    reinterpret_cast<bf16x2*>(base + kFp4RopeOffset + r * kDr * 2)[lane] = rotate_pair(x, cs);
  }
  if ((lane & 3) == 0) reinterpret_cast<unsigned char*>(base + kFp4ScaleOffset + r * (kDc / kMxBlock))[lane >> 2] =
      (unsigned char)(k + 127);
}

// bf16 pages [num_pages, 64, 576] -> 4-bit pages [num_pages, 25600 bytes],
// page for page: one wave per token row.
__global__ __launch_bounds__(256) void quantize_cache_mxfp4_kernel(const char* __restrict__ kv, int64_t num_pages,
                                                                   char* __restrict__ out) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= num_pages * kPage) return;
  const int64_t page = row >> 6;
  const int r = (int)(row & (kPage - 1));
  const char* src = kv + page * kPageBytes + (int64_t)r * kRowBytes;
  char* base = out + page * kFp4PageBytes;
  int k;
  const unsigned codes = quantize_row_mxfp4(reinterpret_cast<const bf16x8*>(src)[lane], k);
  reinterpret_cast<unsigned*>(base + r * kFp4RowBytes)[lane] = codes;
  if (lane < kDr * 2 / 16)
    reinterpret_cast<f32x4*>(base + kFp4RopeOffset + r * kDr * 2)[lane] =
        reinterpret_cast<const f32x4*>(src + kDc * 2)[lane];
  if ((lane & 3) == 0) reinterpret_cast<unsigned char*>(base + kFp4ScaleOffset + r * (kDc / kMxBlock))[lane >> 2] =
      (unsigned char)(k + 127);
}

// q_R [T, H, 64] rotated in place: one thread per 4 pairs (16 bytes). Rows of
// tokens without a position below max_pos are left as they are.
__global__ __launch_bounds__(256) void rope_q_kernel(__bf16* __restrict__ q_r, const float2* __restrict__ rope,
                                                     int max_pos, const int32_t* __restrict__ seqlens, int T,
                                                     int s_q) {
  const int gid = blockIdx.x * 256 + threadIdx.x;  // (t, h, quarter)
  const int quarter = gid & 7;
  const int th = gid >> 3;
  const int t = th / kH;
  if (t >= T) return;
  const int b = t / s_q, i = t - b * s_q;
  const int p = chunk_position(seqlens, b, i, s_q, max_pos);
  if (p < 0) return;
  bf16x8* ptr = reinterpret_cast<bf16x8*>(q_r + (int64_t)th * kDr) + quarter;
  const bf16x8 x = *ptr;
  const float2* cs = rope + (int64_t)p * (kDr / 2) + 4 * quarter;
  bf16x8 y;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x2 r = rotate_pair(bf16x2{x[2 * k], x[2 * k + 1]}, cs[k]);
    y[2 * k] = r[0];
    y[2 * k + 1] = r[1];
  }
  *ptr = y;
}

hipError_t launch_append_latent(const __bf16* c_new, const __bf16* kr_new, const float* rope, int max_pos, char* kv,
                                int64_t num_pages, const int32_t* block_table, int max_pages, const int32_t* seqlens,
                                int B, int s_q, hipStream_t stream) {
  const int T = B * s_q;
  hipLaunchKernelGGL(append_latent_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, c_new, kr_new,
                     reinterpret_cast<const float2*>(rope), max_pos, kv, num_pages, block_table, max_pages, seqlens,
                     T, s_q);
  return hipGetLastError();
}

hipError_t launch_append_latent_fp8(const __bf16* c_new, const __bf16* kr_new, const float* rope, int max_pos,
                                    char* kv, int64_t num_pages, const int32_t* block_table, int max_pages,
                                    const int32_t* seqlens, int B, int s_q, hipStream_t stream) {
  const int T = B * s_q;
  hipLaunchKernelGGL(append_latent_fp8_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, c_new, kr_new,
                     reinterpret_cast<const float2*>(rope), max_pos, kv, num_pages, block_table, max_pages, seqlens,
                     T, s_q);
  return hipGetLastError();
}

hipError_t launch_quantize_cache_fp8(const char* kv, int64_t num_pages, char* out, hipStream_t stream) {
  const int64_t blocks = num_pages * (kPage / 4);
  hipLaunchKernelGGL(quantize_cache_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, kv, num_pages, out);
  return hipGetLastError();
}

hipError_t launch_append_latent_mxfp4(const __bf16* c_new, const __bf16* kr_new, const float* rope, int max_pos,
                                      char* kv, int64_t num_pages, const int32_t* block_table, int max_pages,
                                      const int32_t* seqlens, int B, int s_q, hipStream_t stream) {
  const int T = B * s_q;
  hipLaunchKernelGGL(append_latent_mxfp4_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, c_new, kr_new,
                     reinterpret_cast<const float2*>(rope), max_pos, kv, num_pages, block_table, max_pages, seqlens,
                     T, s_q);
  return hipGetLastError();
}

hipError_t launch_quantize_cache_mxfp4(const char* kv, int64_t num_pages, char* out, hipStream_t stream) {
  const int64_t blocks = num_pages * (kPage / 4);
  hipLaunchKernelGGL(quantize_cache_mxfp4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, kv, num_pages, out);
  return hipGetLastError();
}

hipError_t launch_rope_q(__bf16* q_r, const float* rope, int max_pos, const int32_t* seqlens, int B, int s_q,
                         hipStream_t stream) {
  const int T = B * s_q;
  const int64_t threads = (int64_t)T * kH * 8;
  hipLaunchKernelGGL(rope_q_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, q_r,
                     reinterpret_cast<const float2*>(rope), max_pos, seqlens, T, s_q);
  return hipGetLastError();
}

void rope_table_host(double base, int max_pos, float* table) {
  double theta[kRopePairs];
  for (int j = 0; j < kRopePairs; ++j) theta[j] = std::pow(base, -2.0 * j / (2 * kRopePairs));
  for (int64_t p = 0; p < max_pos; ++p) {
    for (int j = 0; j < kRopePairs; ++j) {
      const double a = (double)p * theta[j];
      table[(p * kRopePairs + j) * 2] = (float)std::cos(a);
      table[(p * kRopePairs + j) * 2 + 1] = (float)std::sin(a);
    }
  }
}

}  // namespace mla
