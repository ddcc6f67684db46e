// Launch interfaces of the MLA kernels (host side of each .hip file).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mla {

struct DecodeParams {
  const __bf16* q_abs;        // [B, s_q, 128, 512]
  const __bf16* q_r;          // [B, s_q, 128, 64]
  const char* kv;             // [num_pages, 64, 576] bf16, or 8-bit / 4-bit pages (launch_decode_paged_fp8 / _mxfp4)
  int64_t num_pages;
  const int32_t* block_table; // [B, max_pages]
  int max_pages;
  const int32_t* seqlens;     // [B]
  int B;
  int s_q;
  int num_splits;
  float scale_log2;           // softmax_scale * log2(e)
  float* o_part;              // [B, s_q, 128, num_splits, 512]
  float* lse_part;            // [B, s_q, 128, num_splits]
};

// cache formats of the scan: bf16 rows, the 8-bit pages of fp8_cache.hpp,
// the 4-bit pages of mxfp4_cache.hpp
constexpr int kFmtBf16 = 0;
constexpr int kFmtFp8 = 1;
constexpr int kFmtMxfp4 = 2;

hipError_t launch_decode_paged(const DecodeParams& p, hipStream_t stream);

// The same scan over the 8-bit cache of fp8_cache.hpp (p.kv: pages of 41216 bytes).
hipError_t launch_decode_paged_fp8(const DecodeParams& p, hipStream_t stream);

// The same scan over the 4-bit cache of mxfp4_cache.hpp (p.kv: pages of 25600 bytes).
hipError_t launch_decode_paged_mxfp4(const DecodeParams& p, hipStream_t stream);

hipError_t launch_combine(const float* o_part, const float* lse_part, int rows, int num_splits,
                          float* o_lat, float* lse, hipStream_t stream);

hipError_t launch_combine_up(const float* o_part, const float* lse_part, const __bf16* w_uv, int T, int num_splits,
                             __bf16* out, float* lse, hipStream_t stream);

hipError_t launch_absorb(const __bf16* q_c, const __bf16* w_uk, __bf16* q_abs, int T, hipStream_t stream);

hipError_t launch_up_proj(const float* o_lat, const __bf16* w_uv, __bf16* out, int T, hipStream_t stream);

hipError_t launch_gather(const char* kv, int64_t num_pages, const int32_t* block_table, int max_pages,
                         const int32_t* seqlens, int B, int max_len, __bf16* out, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, int64_t bytes, float* sink, hipStream_t stream);
hipError_t launch_mfma_loop(int64_t iters, float* sink, hipStream_t stream);

}  // namespace mla
