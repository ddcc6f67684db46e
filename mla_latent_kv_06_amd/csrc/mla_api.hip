// extern "C" entry points of libmla: host-side validation, launch-parameter
// setup and kernel launches. Everything is enqueued on the caller's stream;
// nothing here synchronises or allocates.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/mla.h"
#include "append.hpp"
#include "decode.hpp"
#include "fp8_cache.hpp"
#include "prefill.hpp"
#include "step.hpp"
#include "validate.hpp"

namespace {

thread_local std::string g_last_error;

mla_status report(const mla::Check& c) {
  if (!c.ok()) g_last_error = c.detail;
  return c.status;
}

mla_status report_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return MLA_OK;
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return MLA_ERR_HIP;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// MLA_DEBUG_CHECKS set to anything but "" or "0": the paged scans and steps
// copy the device block table and lengths to the host (synchronously, after
// the caller's stream has drained) and validate them before launching, so a
// bad table is reported instead of being clamped. Debug only: the copy
// allocates host memory and synchronises, and is not capturable.
bool debug_checks() {
  const char* e = std::getenv("MLA_DEBUG_CHECKS");
  return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
}

mla_status debug_table_check(const int32_t* block_table, int max_pages, const int32_t* seqlens, int B,
                             int64_t num_pages, void* stream) {
  std::vector<int32_t> bt((size_t)B * (size_t)max_pages), sl((size_t)B);
  const hipStream_t s = as_stream(stream);
  hipError_t e = hipMemcpyAsync(bt.data(), block_table, bt.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(sl.data(), seqlens, sl.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return report_hip(e, "MLA_DEBUG_CHECKS: block table copy");
  const mla::Check c = mla::validate_block_table(bt.data(), max_pages, sl.data(), B, num_pages, nullptr, nullptr);
  if (!c.ok()) {
    mla::Check d = c;
    d.detail = "MLA_DEBUG_CHECKS: " + c.detail;
    return report(d);
  }
  return MLA_OK;
}

mla_status decode_paged_any(const void* q_abs, const void* q_r, const void* kv_cache, int64_t num_pages,
                            const int32_t* block_table, int max_pages, const int32_t* seqlens, int B, int s_q, int H,
                            float softmax_scale, int num_splits, float* o_part, float* lse_part, void* stream,
                            int fmt) {
  const mla::Check c = mla::check_decode(q_abs, q_r, kv_cache, num_pages, block_table, max_pages, seqlens, B, s_q, H,
                                         softmax_scale, num_splits, o_part, lse_part);
  if (!c.ok()) return report(c);
  if (debug_checks()) {
    const mla_status st = debug_table_check(block_table, max_pages, seqlens, B, num_pages, stream);
    if (st != MLA_OK) return st;
  }
  mla::DecodeParams p{};
  p.q_abs = static_cast<const __bf16*>(q_abs);
  p.q_r = static_cast<const __bf16*>(q_r);
  p.kv = static_cast<const char*>(kv_cache);
  p.num_pages = num_pages;
  p.block_table = block_table;
  p.max_pages = max_pages;
  p.seqlens = seqlens;
  p.B = B;
  p.s_q = s_q;
  p.num_splits = num_splits;
  p.scale_log2 = softmax_scale * 1.44269504088896340736f;
  p.o_part = o_part;
  p.lse_part = lse_part;
  if (fmt == mla::kFmtFp8)
    return report_hip(mla::launch_decode_paged_fp8(p, as_stream(stream)), "mla_decode_paged_fp8 launch");
  if (fmt == mla::kFmtMxfp4)
    return report_hip(mla::launch_decode_paged_mxfp4(p, as_stream(stream)), "mla_decode_paged_mxfp4 launch");
  return report_hip(mla::launch_decode_paged(p, as_stream(stream)), "mla_decode_paged launch");
}

mla_status decode_step_any(const void* q_c, const void* q_r, const void* kv_cache, int64_t num_pages,
                           const int32_t* block_table, int max_pages, const int32_t* seqlens, int B, int s_q, int H,
                           const void* w_uk, const void* w_uv, float softmax_scale, int num_splits, void* q_abs,
                           float* o_part, float* lse_part, float* o_lat, void* out, float* lse, void* stream,
                           int fmt) {
  const mla::Check c = mla::check_step(q_c, q_r, kv_cache, num_pages, block_table, max_pages, seqlens, B, s_q, H, w_uk,
                                       w_uv, softmax_scale, num_splits, q_abs, o_part, lse_part, o_lat, out, lse);
  if (!c.ok()) return report(c);
  if (debug_checks()) {
    const mla_status st = debug_table_check(block_table, max_pages, seqlens, B, num_pages, stream);
    if (st != MLA_OK) return st;
  }
  mla::StepParams p{};
  p.d.q_abs = static_cast<const __bf16*>(q_abs);
  p.d.q_r = static_cast<const __bf16*>(q_r);
  p.d.kv = static_cast<const char*>(kv_cache);
  p.d.num_pages = num_pages;
  p.d.block_table = block_table;
  p.d.max_pages = max_pages;
  p.d.seqlens = seqlens;
  p.d.B = B;
  p.d.s_q = s_q;
  p.d.num_splits = num_splits;
  p.d.scale_log2 = softmax_scale * 1.44269504088896340736f;
  p.d.o_part = o_part;
  p.d.lse_part = lse_part;
  p.q_c = static_cast<const __bf16*>(q_c);
  p.w_uk = static_cast<const __bf16*>(w_uk);
  p.w_uv = static_cast<const __bf16*>(w_uv);
  p.o_lat = o_lat;
  p.lse = lse;
  p.out = static_cast<__bf16*>(out);
  return report_hip(mla::launch_decode_step(p, fmt, as_stream(stream)),
                    fmt == mla::kFmtFp8     ? "mla_decode_step_fp8 launch"
                    : fmt == mla::kFmtMxfp4 ? "mla_decode_step_mxfp4 launch"
                                            : "mla_decode_step launch");
}

}  // namespace

// detail for mla_last_error from entry points defined in other sources
void mla_set_last_error(const std::string& s) { g_last_error = s; }

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    default: return "MLA_ERR_UNKNOWN";
  }
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

mla_status mla_validate_block_table(const int32_t* block_table, int max_pages, const int32_t* seqlens, int B,
                                    int64_t num_pages, int* bad_seq, int* bad_page) {
  return report(mla::validate_block_table(block_table, max_pages, seqlens, B, num_pages, bad_seq, bad_page));
}

size_t mla_decode_workspace_bytes(int B, int s_q, int H, int num_splits) {
  return mla::workspace_bytes(B, s_q, H, num_splits);
}

int mla_recommended_splits(int B, int s_q, int max_len, int num_cus) {
  return mla::recommended_splits(B, s_q, max_len, num_cus);
}

int mla_plan_splits(const int32_t* seqlens_host, int B, int s_q, int max_pages, int num_cus) {
  return mla::plan_splits(seqlens_host, B, s_q, max_pages, num_cus);
}

mla_status mla_absorb_q(const void* q_c, const void* w_uk, void* q_abs, int64_t T, int H, void* stream) {
  const mla::Check c = mla::check_absorb(q_c, w_uk, q_abs, T, H);
  if (!c.ok()) return report(c);
  return report_hip(mla::launch_absorb(static_cast<const __bf16*>(q_c), static_cast<const __bf16*>(w_uk),
                                       static_cast<__bf16*>(q_abs), (int)T, as_stream(stream)),
                    "mla_absorb_q launch");
}

mla_status mla_decode_paged(const void* q_abs, const void* q_r, const void* kv_cache, int64_t num_pages,
                            const int32_t* block_table, int max_pages, const int32_t* seqlens, int B, int s_q,
                            int H, float softmax_scale, int num_splits, float* o_part, float* lse_part,
                            void* stream) {
  return decode_paged_any(q_abs, q_r, kv_cache, num_pages, block_table, max_pages, seqlens, B, s_q, H, softmax_scale,
                          num_splits, o_part, lse_part, stream, mla::kFmtBf16);
}


mla_status mla_decode_paged_fp8(const void* q_abs, const void* q_r, const void* kv_fp8, int64_t num_pages,
                                const int32_t* block_table, int max_pages, const int32_t* seqlens, int B, int s_q,
                                int H, float softmax_scale, int num_splits, float* o_part, float* lse_part,
                                void* stream) {
  return decode_paged_any(q_abs, q_r, kv_fp8, num_pages, block_table, max_pages, seqlens, B, s_q, H, softmax_scale,
                          num_splits, o_part, lse_part, stream, mla::kFmtFp8);
}

mla_status mla_quantize_cache_fp8(const void* kv_cache, int64_t num_pages, void* kv_fp8, void* stream) {
  const mla::Check c = mla::check_quantize_cache(kv_cache, num_pages, kv_fp8);
  if (!c.ok()) return report(c);
  return report_hip(mla::launch_quantize_cache_fp8(static_cast<const char*>(kv_cache), num_pages,
                                                   static_cast<char*>(kv_fp8), as_stream(stream)),
                    "mla_quantize_cache_fp8 launch");
}

mla_status mla_append_latent_fp8(const void* c_new, const void* kr_new, const float* rope, int max_pos, void* kv_fp8,
                                 int64_t num_pages, const int32_t* block_table, int max_pages, const int32_t* seqlens,
                                 int B, int s_q, void* stream) {
  const mla::Check c = mla::check_append(c_new, kr_new, rope, max_pos, kv_fp8, num_pages, block_table, max_pages,
                                         seqlens, B, s_q);
  if (!c.ok()) return report(c);
  return report_hip(mla::launch_append_latent_fp8(static_cast<const __bf16*>(c_new),
                                                  static_cast<const __bf16*>(kr_new), rope, max_pos,
                                                  static_cast<char*>(kv_fp8), num_pages, block_table, max_pages,
                                                  seqlens, B, s_q, as_stream(stream)),
                    "mla_append_latent_fp8 launch");
}

mla_status mla_decode_paged_mxfp4(const void* q_abs, const void* q_r, const void* kv_fp4, int64_t num_pages,
                                  const int32_t* block_table, int max_pages, const int32_t* seqlens, int B, int s_q,
                                  int H, float softmax_scale, int num_splits, float* o_part, float* lse_part,
                                  void* stream) {
  return decode_paged_any(q_abs, q_r, kv_fp4, num_pages, block_table, max_pages, seqlens, B, s_q, H, softmax_scale,
                          num_splits, o_part, lse_part, stream, mla::kFmtMxfp4);
}

mla_status mla_quantize_cache_mxfp4(const void* kv_cache, int64_t num_pages, void* kv_fp4, void* stream) {
  const mla::Check c = mla::check_quantize_cache(kv_cache, num_pages, kv_fp4);
  if (!c.ok()) return report(c);
  return report_hip(mla::launch_quantize_cache_mxfp4(static_cast<const char*>(kv_cache), num_pages,
                                                     static_cast<char*>(kv_fp4), as_stream(stream)),
                    "mla_quantize_cache_mxfp4 launch");
}

mla_status mla_append_latent_mxfp4(const void* c_new, const void* kr_new, const float* rope, int max_pos,
                                   void* kv_fp4, int64_t num_pages, const int32_t* block_table, int max_pages,
                                   const int32_t* seqlens, int B, int s_q, void* stream) {
  const mla::Check c = mla::check_append(c_new, kr_new, rope, max_pos, kv_fp4, num_pages, block_table, max_pages,
                                         seqlens, B, s_q);
  if (!c.ok()) return report(c);
  return report_hip(mla::launch_append_latent_mxfp4(static_cast<const __bf16*>(c_new),
                                                    static_cast<const __bf16*>(kr_new), rope, max_pos,
                                                    static_cast<char*>(kv_fp4), num_pages, block_table, max_pages,
                                                    seqlens, B, s_q, as_stream(stream)),
                    "mla_append_latent_mxfp4 launch");
}

mla_status mla_decode_step(const void* q_c, const void* q_r, const void* kv_cache, int64_t num_pages,
                           const int32_t* block_table, int max_pages, const int32_t* seqlens, int B, int s_q, int H,
                           const void* w_uk, const void* w_uv, float softmax_scale, int num_splits, void* q_abs,
                           float* o_part, float* lse_part, float* o_lat, void* out, float* lse, void* stream) {
  return decode_step_any(q_c, q_r, kv_cache, num_pages, block_table, max_pages, seqlens, B, s_q, H, w_uk, w_uv,
                         softmax_scale, num_splits, q_abs, o_part, lse_part, o_lat, out, lse, stream, mla::kFmtBf16);
}

mla_status mla_decode_step_fp8(const void* q_c, const void* q_r, const void* kv_fp8, int64_t num_pages,
                               const int32_t* block_table, int max_pages, const int32_t* seqlens, int B, int s_q,
                               int H, const void* w_uk, const void* w_uv, float softmax_scale, int num_splits,
                               void* q_abs, float* o_part, float* lse_part, float* o_lat, void* out, float* lse,
                               void* stream) {
  return decode_step_any(q_c, q_r, kv_fp8, num_pages, block_table, max_pages, seqlens, B, s_q, H, w_uk, w_uv,
                         softmax_scale, num_splits, q_abs, o_part, lse_part, o_lat, out, lse, stream, mla::kFmtFp8);
}

mla_status mla_decode_step_mxfp4(const void* q_c, const void* q_r, const void* kv_fp4, int64_t num_pages,
                                 const int32_t* block_table, int max_pages, const int32_t* seqlens, int B, int s_q,
                                 int H, const void* w_uk, const void* w_uv, float softmax_scale, int num_splits,
                                 void* q_abs, float* o_part, float* lse_part, float* o_lat, void* out, float* lse,
                                 void* stream) {
  return decode_step_any(q_c, q_r, kv_fp4, num_pages, block_table, max_pages, seqlens, B, s_q, H, w_uk, w_uv,
                         softmax_scale, num_splits, q_abs, o_part, lse_part, o_lat, out, lse, stream, mla::kFmtMxfp4);
}

mla_status mla_combine_splits(const float* o_part, const float* lse_part, int B, int s_q, int H, int num_splits,
                              float* o_lat, float* lse, void* stream) {
  const mla::Check c = mla::check_combine(o_part, lse_part, B, s_q, H, num_splits, o_lat, lse);
  if (!c.ok()) return report(c);
  return report_hip(mla::launch_combine(o_part, lse_part, B * s_q * H, num_splits, o_lat, lse, as_stream(stream)),
                    "mla_combine_splits launch");
}

mla_status mla_combine_up_proj(const float* o_part, const float* lse_part, const void* w_uv, int B, int s_q, int H,
                               int num_splits, void* out, float* lse, void* stream) {
  const mla::Check c = mla::check_combine_up(o_part, lse_part, w_uv, B, s_q, H, num_splits, out, lse);
  if (!c.ok()) return report(c);
  return report_hip(mla::launch_combine_up(o_part, lse_part, static_cast<const __bf16*>(w_uv), B * s_q, num_splits,
                                           static_cast<__bf16*>(out), lse, as_stream(stream)),
                    "mla_combine_up_proj launch");
}

mla_status mla_up_proj(const float* o_lat, const void* w_uv, void* out, int64_t T, int H, void* stream) {
  const mla::Check c = mla::check_up_proj(o_lat, w_uv, out, T, H);
  if (!c.ok()) return report(c);
  return report_hip(mla::launch_up_proj(o_lat, static_cast<const __bf16*>(w_uv), static_cast<__bf16*>(out), (int)T,
                                        as_stream(stream)),
                    "mla_up_proj launch");
}

mla_status mla_rope_table(double base, int max_pos, float* table) {
  const mla::Check c = mla::check_rope_table(base, max_pos, table, mla::kMaxRopePositions);
  if (!c.ok()) return report(c);
  mla::rope_table_host(base, max_pos, table);
  return MLA_OK;
}

mla_status mla_append_latent(const void* c_new, const void* kr_new, const float* rope, int max_pos, void* kv_cache,
                             int64_t num_pages, const int32_t* block_table, int max_pages, const int32_t* seqlens,
                             int B, int s_q, void* stream) {
  const mla::Check c = mla::check_append(c_new, kr_new, rope, max_pos, kv_cache, num_pages, block_table, max_pages,
                                         seqlens, B, s_q);
  if (!c.ok()) return report(c);
  return report_hip(mla::launch_append_latent(static_cast<const __bf16*>(c_new), static_cast<const __bf16*>(kr_new),
                                              rope, max_pos, static_cast<char*>(kv_cache), num_pages, block_table,
                                              max_pages, seqlens, B, s_q, as_stream(stream)),
                    "mla_append_latent launch");
}

mla_status mla_rope_q(void* q_r, const float* rope, int max_pos, const int32_t* seqlens, int B, int s_q, int H,
                      void* stream) {
  const mla::Check c = mla::check_rope_q(q_r, rope, max_pos, seqlens, B, s_q, H);
  if (!c.ok()) return report(c);
  return report_hip(mla::launch_rope_q(static_cast<__bf16*>(q_r), rope, max_pos, seqlens, B, s_q, as_stream(stream)),
                    "mla_rope_q launch");
}

int mla_prefill_uses_absorption(int s_q) { return s_q <= mla::kPrefillAbsorptionThreshold ? 1 : 0; }

size_t mla_decompressed_kv_bytes(int B, int max_len) {
  if (B <= 0 || max_len <= 0) return 0;
  return (size_t)B * MLA_HEADS * (size_t)max_len * MLA_D_HC * 2;
}

mla_status mla_decompress_kv(const void* kv_cache, int64_t num_pages, const int32_t* block_table, int max_pages,
                             const int32_t* seqlens, int B, int max_len, const void* w_uk, const void* w_uv,
                             void* k_nope, void* v, void* stream) {
  const mla::Check c = mla::check_decompress(kv_cache, num_pages, block_table, max_pages, seqlens, B, max_len, w_uk,
                                             w_uv, k_nope, v);
  if (!c.ok()) return report(c);
  return report_hip(mla::launch_decompress_kv(static_cast<const char*>(kv_cache), num_pages, block_table, max_pages,
                                              seqlens, B, max_len, static_cast<const __bf16*>(w_uk),
                                              static_cast<const __bf16*>(w_uv), static_cast<__bf16*>(k_nope),
                                              static_cast<_Float16*>(v), as_stream(stream)),
                    "mla_decompress_kv launch");
}

mla_status mla_prefill_mha(const void* q_c, const void* q_r, const void* k_nope, const void* v, int max_len,
                           const void* kv_cache, int64_t num_pages, const int32_t* block_table, int max_pages,
                           const int32_t* seqlens, int B, int s_q, int H, float softmax_scale, void* out, float* lse,
                           void* stream) {
  const mla::Check c = mla::check_prefill_mha(q_c, q_r, k_nope, v, max_len, kv_cache, num_pages, block_table,
                                              max_pages, seqlens, B, s_q, H, softmax_scale, out, lse);
  if (!c.ok()) return report(c);
  return report_hip(mla::launch_prefill_mha(static_cast<const __bf16*>(q_c), static_cast<const __bf16*>(q_r),
                                            static_cast<const __bf16*>(k_nope), static_cast<const _Float16*>(v), max_len,
                                            static_cast<const char*>(kv_cache), num_pages, block_table, max_pages,
                                            seqlens, B, s_q, softmax_scale * 1.44269504088896340736f,
                                            static_cast<__bf16*>(out), lse, as_stream(stream)),
                    "mla_prefill_mha launch");
}

mla_status mla_debug_gather(const void* kv_cache, int64_t num_pages, const int32_t* block_table, int max_pages,
                            const int32_t* seqlens, int B, int max_len, void* out, void* stream) {
  const mla::Check c = mla::check_gather(kv_cache, num_pages, block_table, max_pages, seqlens, B, max_len, out);
  if (!c.ok()) return report(c);
  return report_hip(mla::launch_gather(static_cast<const char*>(kv_cache), num_pages, block_table, max_pages, seqlens,
                                       B, max_len, static_cast<__bf16*>(out), as_stream(stream)),
                    "mla_debug_gather launch");
}

mla_status mla_bench_stream_read(const void* buf, int64_t bytes, float* sink, void* stream) {
  const mla::Check c = mla::check_bench_stream_read(buf, bytes, sink);
  if (!c.ok()) return report(c);
  return report_hip(mla::launch_stream_read(buf, bytes, sink, as_stream(stream)), "mla_bench_stream_read launch");
}

mla_status mla_bench_mfma(int64_t iters, float* sink, void* stream) {
  const mla::Check c = mla::check_bench_mfma(iters, sink);
  if (!c.ok()) return report(c);
  return report_hip(mla::launch_mfma_loop(iters, sink, as_stream(stream)), "mla_bench_mfma launch");
}

}  // extern "C"
