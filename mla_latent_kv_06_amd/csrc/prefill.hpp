// Launch interfaces of the decompressed branch (decompress.hip, prefill_mha.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mla {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kPrefillAbsorptionThreshold = 256;  // chunks up to this many new tokens stay absorbed

// K [B, 128, max_len, 128] bf16 and V (same shape) fp16: rows t < L_b of
// each (b, h), zeros up to the end of L_b's page; later rows untouched.
hipError_t launch_decompress_kv(const char* kv, int64_t num_pages, const int32_t* block_table, int max_pages,
                                const int32_t* seqlens, int B, int max_len, const __bf16* w_uk, const __bf16* w_uv,
                                __bf16* k_out, _Float16* v_out, hipStream_t stream);

// out [B, s_q, 128, 128] bf16 and lse [B, s_q, 128] fp32 over the K, V of
// launch_decompress_kv (max_len a multiple of 64) and the cache's k_R.
hipError_t launch_prefill_mha(const __bf16* q_c, const __bf16* q_r, const __bf16* k_nope, const _Float16* v, int max_len,
                              const char* kv, int64_t num_pages, const int32_t* block_table, int max_pages,
                              const int32_t* seqlens, int B, int s_q, float scale_log2, __bf16* out, float* lse,
                              hipStream_t stream);

}  // namespace mla
