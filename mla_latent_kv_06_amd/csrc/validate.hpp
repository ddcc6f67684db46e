// Host-side argument checks and split planning for the MLA C ABI.
// Plain C++17 with no HIP dependency, so it compiles and is unit-tested with
// g++ on a machine without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/mla.h"

namespace mla {

constexpr int kMaxSq = 4096;

struct Check {
  mla_status status = MLA_OK;
  std::string detail;
  bool ok() const { return status == MLA_OK; }
};

inline Check fail(mla_status s, const char* fmt, const char* a = "", long long v = 0) {
  Check c;
  c.status = s;
  char buf[256];
  std::snprintf(buf, sizeof buf, fmt, a, v);
  c.detail = buf;
  return c;
}

inline Check need_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(MLA_ERR_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(MLA_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return Check{};
}

inline Check need_range(long long v, long long lo, long long hi, const char* name) {
  if (v < lo || v > hi) {
    Check c;
    c.status = MLA_ERR_SHAPE;
    char buf[256];
    std::snprintf(buf, sizeof buf, "%s = %lld outside [%lld, %lld]", name, v, lo, hi);
    c.detail = buf;
    return c;
  }
  return Check{};
}

#define MLA_TRY(expr)            \
  do {                           \
    ::mla::Check _c = (expr);    \
    if (!_c.ok()) return _c;     \
  } while (0)

inline Check check_absorb(const void* q_c, const void* w_uk, const void* q_abs, int64_t T, int H) {
  MLA_TRY(need_ptr(q_c, "q_c"));
  MLA_TRY(need_ptr(w_uk, "w_uk"));
  MLA_TRY(need_ptr(q_abs, "q_abs"));
  MLA_TRY(need_range(T, 1, (1LL << 31) / MLA_HEADS, "T"));
  MLA_TRY(need_range(H, MLA_HEADS, MLA_HEADS, "H"));
  return Check{};
}

inline Check check_up_proj(const void* o_lat, const void* w_uv, const void* out, int64_t T, int H) {
  MLA_TRY(need_ptr(o_lat, "o_lat"));
  MLA_TRY(need_ptr(w_uv, "w_uv"));
  MLA_TRY(need_ptr(out, "out"));
  MLA_TRY(need_range(T, 1, (1LL << 31) / MLA_HEADS, "T"));
  MLA_TRY(need_range(H, MLA_HEADS, MLA_HEADS, "H"));
  return Check{};
}

inline Check check_decode(const void* q_abs, const void* q_r, const void* kv, int64_t num_pages,
                          const void* bt, int max_pages, const void* seqlens, int B, int s_q, int H,
                          float scale, int num_splits, const void* o_part, const void* lse_part) {
  MLA_TRY(need_ptr(q_abs, "q_abs"));
  MLA_TRY(need_ptr(q_r, "q_r"));
  MLA_TRY(need_ptr(kv, "kv_cache"));
  MLA_TRY(need_ptr(bt, "block_table"));
  MLA_TRY(need_ptr(seqlens, "seqlens"));
  MLA_TRY(need_ptr(o_part, "o_part"));
  MLA_TRY(need_ptr(lse_part, "lse_part"));
  MLA_TRY(need_range(num_pages, 1, (1LL << 40), "num_pages"));
  MLA_TRY(need_range(max_pages, 1, (1 << 24), "max_pages"));
  MLA_TRY(need_range(B, 1, (1 << 20), "B"));
  MLA_TRY(need_range(s_q, 1, kMaxSq, "s_q"));
  MLA_TRY(need_range(H, MLA_HEADS, MLA_HEADS, "H"));
  MLA_TRY(need_range(num_splits, 1, max_pages, "num_splits"));
  if (!(scale > 0.0f) || scale > 3.0e38f)
    return fail(MLA_ERR_SHAPE, "softmax_scale must be positive and finite%s", "");
  // grid size: work items are (b, i, split); keep well inside 32-bit counts
  long long items = (long long)B * s_q * num_splits;
  MLA_TRY(need_range(items, 1, (1LL << 30), "B * s_q * num_splits"));
  // partial rows index o_part with 64-bit offsets; nothing more to check here
  return Check{};
}

inline Check check_combine(const void* o_part, const void* lse_part, int B, int s_q, int H,
                           int num_splits, const void* o_lat, const void* lse) {
  MLA_TRY(need_ptr(o_part, "o_part"));
  MLA_TRY(need_ptr(lse_part, "lse_part"));
  MLA_TRY(need_ptr(o_lat, "o_lat"));
  MLA_TRY(need_ptr(lse, "lse"));
  MLA_TRY(need_range(B, 1, (1 << 20), "B"));
  MLA_TRY(need_range(s_q, 1, kMaxSq, "s_q"));
  MLA_TRY(need_range(H, MLA_HEADS, MLA_HEADS, "H"));
  MLA_TRY(need_range(num_splits, 1, (1 << 16), "num_splits"));
  MLA_TRY(need_range((long long)B * s_q * H, 1, (1LL << 31) - 1, "B * s_q * H"));
  return Check{};
}

inline Check check_gather(const void* kv, int64_t num_pages, const void* bt, int max_pages,
                          const void* seqlens, int B, int max_len, const void* out) {
  MLA_TRY(need_ptr(kv, "kv_cache"));
  MLA_TRY(need_ptr(bt, "block_table"));
  MLA_TRY(need_ptr(seqlens, "seqlens"));
  MLA_TRY(need_ptr(out, "out"));
  MLA_TRY(need_range(num_pages, 1, (1LL << 40), "num_pages"));
  MLA_TRY(need_range(max_pages, 1, (1 << 24), "max_pages"));
  MLA_TRY(need_range(B, 1, (1 << 20), "B"));
  MLA_TRY(need_range(max_len, 1, (1 << 26), "max_len"));
  return Check{};
}

inline size_t workspace_bytes(int B, int s_q, int H, int num_splits) {
  if (B < 1 || s_q < 1 || H < 1 || num_splits < 1) return 0;
  return (size_t)B * s_q * H * num_splits * (MLA_D_C + 1) * sizeof(float);
}

// Split count: enough (b, i, split) work items for about two per compute
// unit, but never splits shorter than kMinSplitPages pages, because each
// split writes a 256 KiB partial that costs as much HBM time as reading
// ~3.5 pages of cache.
inline int recommended_splits(int B, int s_q, int max_len, int num_cus) {
  constexpr int kMinSplitPages = 8;
  if (max_len < 1 || B < 1 || s_q < 1) return 1;
  long long pages = (max_len + MLA_PAGE - 1) / MLA_PAGE;
  long long items = (long long)B * s_q;
  long long cus = num_cus > 0 ? num_cus : 256;
  long long want = (cus + items - 1) / items;  // one work item per CU
  long long cap = pages / kMinSplitPages;
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want > pages) want = pages;
  if (want < 1) want = 1;
  return (int)want;
}

}  // namespace mla
