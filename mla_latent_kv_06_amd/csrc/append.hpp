// Launch interfaces of the cache-append and RoPE kernels (append.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mla {

constexpr int kRopePairs = 32;            // pairs of the 64-value RoPE part
constexpr int kMaxRopePositions = 1 << 22;  // table rows the host helper builds at most (1 GiB)

// Chunk token (b, i) -> cache row L_b - s_q + i: c_KV copied, k_R rotated.
hipError_t launch_append_latent(const __bf16* c_new, const __bf16* kr_new, const float* rope, int max_pos, char* kv,
                                int64_t num_pages, const int32_t* block_table, int max_pages, const int32_t* seqlens,
                                int B, int s_q, hipStream_t stream);

// The same append into the 8-bit cache (fp8_cache.hpp): c_KV quantized, k_R rotated.
hipError_t launch_append_latent_fp8(const __bf16* c_new, const __bf16* kr_new, const float* rope, int max_pos,
                                    char* kv, int64_t num_pages, const int32_t* block_table, int max_pages,
                                    const int32_t* seqlens, int B, int s_q, hipStream_t stream);

// bf16 pages -> 8-bit pages, page for page (num_pages * 16 workgroups).
hipError_t launch_quantize_cache_fp8(const char* kv, int64_t num_pages, char* out, hipStream_t stream);
// The same append into the 4-bit cache (mxfp4_cache.hpp), and the page-for-page conversion.
hipError_t launch_append_latent_mxfp4(const __bf16* c_new, const __bf16* kr_new, const float* rope, int max_pos,
                                      char* kv, int64_t num_pages, const int32_t* block_table, int max_pages,
                                      const int32_t* seqlens, int B, int s_q, hipStream_t stream);
hipError_t launch_quantize_cache_mxfp4(const char* kv, int64_t num_pages, char* out, hipStream_t stream);

// q_R [B*s_q, 128, 64] rotated in place by each token's position.
hipError_t launch_rope_q(__bf16* q_r, const float* rope, int max_pos, const int32_t* seqlens, int B, int s_q,
                         hipStream_t stream);

// cos/sin(p * base^(-2j/64)) for p < max_pos, j < 32, computed in double and
// rounded to float: table[(p * 32 + j) * 2 + {0, 1}].
void rope_table_host(double base, int max_pos, float* table);

}  // namespace mla
