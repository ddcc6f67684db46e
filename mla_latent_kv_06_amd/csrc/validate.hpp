// Host-side argument checks and split planning for the MLA C ABI.
// Plain C++17 with no HIP dependency, so it compiles and is unit-tested with
// g++ on a machine without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

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
  // the split plan counts the pages of all rows in 32 bits
  MLA_TRY(need_range((long long)B * s_q * max_pages, 1, (1LL << 31) - 1, "B * s_q * max_pages"));
  // partial rows index o_part with 64-bit offsets; nothing more to check here
  return Check{};
}

inline Check check_step(const void* q_c, const void* q_r, const void* kv, int64_t num_pages, const void* bt,
                        int max_pages, const void* seqlens, int B, int s_q, int H, const void* w_uk,
                        const void* w_uv, float scale, int num_splits, const void* q_abs, const void* o_part,
                        const void* lse_part, const void* o_lat, const void* out, const void* lse) {
  MLA_TRY(need_ptr(q_c, "q_c"));
  MLA_TRY(need_ptr(w_uk, "w_uk"));
  MLA_TRY(need_ptr(w_uv, "w_uv"));
  MLA_TRY(need_ptr(o_lat, "o_lat"));
  MLA_TRY(need_ptr(out, "out"));
  MLA_TRY(need_ptr(lse, "lse"));
  MLA_TRY(check_decode(q_abs, q_r, kv, num_pages, bt, max_pages, seqlens, B, s_q, H, scale, num_splits, o_part,
                       lse_part));
  MLA_TRY(need_range((long long)B * s_q, 1, (1LL << 20), "B * s_q"));
  return Check{};
}

// The allocation-free step keeps q_abs and the split partials in a static
// device array of kStaticScratchBytes; scratch_layout gives each region's
// byte offset (each 256-byte aligned) and the total.
constexpr size_t kStaticScratchBytes = size_t(96) << 20;

struct ScratchLayout {
  size_t q_abs = 0, o_part = 0, lse_part = 0, total = 0;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline ScratchLayout scratch_layout(int B, int s_q, int num_splits) {
  ScratchLayout L;
  const size_t rows = (size_t)B * (size_t)s_q * MLA_HEADS;
  L.q_abs = 0;
  L.o_part = align256(rows * MLA_D_C * 2);
  L.lse_part = L.o_part + align256(rows * (size_t)num_splits * MLA_D_C * 4);
  L.total = L.lse_part + align256(rows * (size_t)num_splits * 4);
  return L;
}

inline Check check_step_static(const void* q_c, const void* q_r, const void* kv, int64_t num_pages, const void* bt,
                               int max_pages, const void* seqlens, int B, int s_q, int H, const void* w_uk,
                               const void* w_uv, float scale, int num_splits, const void* out, const void* lse) {
  MLA_TRY(need_ptr(q_c, "q_c"));
  MLA_TRY(need_ptr(w_uk, "w_uk"));
  MLA_TRY(need_ptr(w_uv, "w_uv"));
  MLA_TRY(need_ptr(out, "out"));
  MLA_TRY(need_ptr(lse, "lse"));
  // q_abs and the partials live in the scratch array; any aligned stand-in
  // passes the pointer checks of the scan
  const void* const inside = reinterpret_cast<const void*>(uintptr_t(256));
  MLA_TRY(check_decode(inside, q_r, kv, num_pages, bt, max_pages, seqlens, B, s_q, H, scale, num_splits, inside,
                       inside));
  MLA_TRY(need_range((long long)B * s_q, 1, (1LL << 20), "B * s_q"));
  const ScratchLayout L = scratch_layout(B, s_q, num_splits);
  if (L.total > kStaticScratchBytes) {
    Check c;
    c.status = MLA_ERR_WORKSPACE;
    char buf[256];
    std::snprintf(buf, sizeof buf,
                  "B * s_q = %lld with num_splits = %d needs %zu bytes of scratch; the static array holds %zu",
                  (long long)B * s_q, num_splits, L.total, kStaticScratchBytes);
    c.detail = buf;
    return c;
  }
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

inline Check check_combine_up(const void* o_part, const void* lse_part, const void* w_uv, int B, int s_q, int H,
                              int num_splits, const void* out, const void* lse) {
  MLA_TRY(check_combine(o_part, lse_part, B, s_q, H, num_splits, out, lse));
  MLA_TRY(need_ptr(w_uv, "w_uv"));
  return Check{};
}

inline Check check_rope_table(double base, int max_pos, const void* table, int max_positions) {
  if (table == nullptr) return fail(MLA_ERR_NULL, "%s is NULL", "table");
  if (!(base > 0.0) || base > 1e300) return fail(MLA_ERR_SHAPE, "%s must be positive and finite", "base");
  MLA_TRY(need_range(max_pos, 1, max_positions, "max_pos"));
  return Check{};
}

inline Check check_append(const void* c_new, const void* kr_new, const void* rope, int max_pos, const void* kv,
                          int64_t num_pages, const void* bt, int max_pages, const void* seqlens, int B, int s_q) {
  MLA_TRY(need_ptr(c_new, "c_new"));
  MLA_TRY(need_ptr(kr_new, "kr_new"));
  MLA_TRY(need_ptr(rope, "rope"));
  MLA_TRY(need_ptr(kv, "kv_cache"));
  MLA_TRY(need_ptr(bt, "block_table"));
  MLA_TRY(need_ptr(seqlens, "seqlens"));
  MLA_TRY(need_range(max_pos, 1, (1LL << 31) - 1, "max_pos"));
  MLA_TRY(need_range(num_pages, 1, (1LL << 40), "num_pages"));
  MLA_TRY(need_range(max_pages, 1, (1 << 24), "max_pages"));
  MLA_TRY(need_range(B, 1, (1 << 20), "B"));
  MLA_TRY(need_range(s_q, 1, kMaxSq, "s_q"));
  MLA_TRY(need_range((long long)B * s_q, 1, (1LL << 24), "B * s_q"));
  return Check{};
}

inline Check check_quantize_cache(const void* kv, int64_t num_pages, const void* out) {
  MLA_TRY(need_ptr(kv, "kv_cache"));
  MLA_TRY(need_ptr(out, "kv_fp8"));
  MLA_TRY(need_range(num_pages, 1, (1LL << 26), "num_pages"));
  return Check{};
}

inline Check check_rope_q(const void* q_r, const void* rope, int max_pos, const void* seqlens, int B, int s_q,
                          int H) {
  MLA_TRY(need_ptr(q_r, "q_r"));
  MLA_TRY(need_ptr(rope, "rope"));
  MLA_TRY(need_ptr(seqlens, "seqlens"));
  MLA_TRY(need_range(max_pos, 1, (1LL << 31) - 1, "max_pos"));
  MLA_TRY(need_range(B, 1, (1 << 20), "B"));
  MLA_TRY(need_range(s_q, 1, kMaxSq, "s_q"));
  MLA_TRY(need_range(H, MLA_HEADS, MLA_HEADS, "H"));
  MLA_TRY(need_range((long long)B * s_q, 1, (1LL << 21), "B * s_q"));
  return Check{};
}

inline Check check_decompress(const void* kv, int64_t num_pages, const void* bt, int max_pages, const void* seqlens,
                              int B, int max_len, const void* w_uk, const void* w_uv, const void* k, const void* v) {
  MLA_TRY(need_ptr(kv, "kv_cache"));
  MLA_TRY(need_ptr(bt, "block_table"));
  MLA_TRY(need_ptr(seqlens, "seqlens"));
  MLA_TRY(need_ptr(w_uk, "w_uk"));
  MLA_TRY(need_ptr(w_uv, "w_uv"));
  MLA_TRY(need_ptr(k, "k_nope"));
  MLA_TRY(need_ptr(v, "v"));
  MLA_TRY(need_range(num_pages, 1, (1LL << 40), "num_pages"));
  MLA_TRY(need_range(max_pages, 1, (1 << 24), "max_pages"));
  MLA_TRY(need_range(B, 1, (1 << 20), "B"));
  MLA_TRY(need_range(max_len, 1, (1 << 30), "max_len"));
  if (max_len % MLA_PAGE != 0) return fail(MLA_ERR_SHAPE, "%s must be a multiple of 64 (got %lld)", "max_len", max_len);
  MLA_TRY(need_range((long long)B * max_len, 1, (1LL << 31), "B * max_len"));
  return Check{};
}

inline Check check_prefill_mha(const void* q_c, const void* q_r, const void* k, const void* v, int max_len,
                               const void* kv, int64_t num_pages, const void* bt, int max_pages, const void* seqlens,
                               int B, int s_q, int H, float scale, const void* out, const void* lse) {
  MLA_TRY(need_ptr(q_c, "q_c"));
  MLA_TRY(need_ptr(q_r, "q_r"));
  MLA_TRY(need_ptr(out, "out"));
  MLA_TRY(need_ptr(lse, "lse"));
  MLA_TRY(need_ptr(k, "k_nope"));
  MLA_TRY(need_ptr(v, "v"));
  MLA_TRY(need_ptr(kv, "kv_cache"));
  MLA_TRY(need_ptr(bt, "block_table"));
  MLA_TRY(need_ptr(seqlens, "seqlens"));
  MLA_TRY(need_range(num_pages, 1, (1LL << 40), "num_pages"));
  MLA_TRY(need_range(max_pages, 1, (1 << 24), "max_pages"));
  MLA_TRY(need_range(B, 1, (1 << 20), "B"));
  MLA_TRY(need_range(max_len, 1, (1 << 30), "max_len"));
  if (max_len % MLA_PAGE != 0) return fail(MLA_ERR_SHAPE, "%s must be a multiple of 64 (got %lld)", "max_len", max_len);
  MLA_TRY(need_range(s_q, 1, (1 << 20), "s_q"));
  MLA_TRY(need_range(H, MLA_HEADS, MLA_HEADS, "H"));
  MLA_TRY(need_range((long long)B * s_q, 1, (1LL << 24), "B * s_q"));
  if (!(scale > 0.f) || scale > 3.0e38f) return fail(MLA_ERR_SHAPE, "%s must be positive and finite", "softmax_scale");
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

inline Check check_bench_stream_read(const void* buf, int64_t bytes, const void* sink) {
  MLA_TRY(need_ptr(buf, "buf"));
  MLA_TRY(need_ptr(sink, "sink"));
  MLA_TRY(need_range(bytes, 16, (1LL << 46), "bytes"));
  if (bytes % 16 != 0) return fail(MLA_ERR_SHAPE, "%s = %lld is not a multiple of 16", "bytes", (long long)bytes);
  return Check{};
}

inline Check check_bench_mfma(int64_t iters, const void* sink) {
  MLA_TRY(need_ptr(sink, "sink"));
  MLA_TRY(need_range(iters, 1, (1LL << 40), "iters"));
  return Check{};
}

// ---- block-table contract ------------------------------------------------
// The decode, gather, append and decompression kernels read entry
// block_table[b, p] for the logical pages p < ceil(L_b / 64) of every
// sequence and clamp each entry into [0, num_pages) on the device, so a bad
// entry never leaves the cache but silently yields another page's rows. This
// host check reports the first entry (in (b, p) order) that breaks the
// contract instead, and lengths outside [0, max_pages * 64] (the kernels clamp
// those too). Entries past a sequence's pages are never read and may hold
// anything (-1 by convention). bad_seq / bad_page (either may be NULL)
// receive the offending sequence and logical page, or page -1 when the length
// itself is out of range; both are -1 when the table is valid.
inline Check validate_block_table(const int32_t* bt, int max_pages, const int32_t* seqlens, int B,
                                  int64_t num_pages, int* bad_seq, int* bad_page) {
  if (bad_seq) *bad_seq = -1;
  if (bad_page) *bad_page = -1;
  if (bt == nullptr) return fail(MLA_ERR_NULL, "%s is NULL", "block_table");
  if (seqlens == nullptr) return fail(MLA_ERR_NULL, "%s is NULL", "seqlens");
  MLA_TRY(need_range(num_pages, 1, (1LL << 40), "num_pages"));
  MLA_TRY(need_range(max_pages, 1, (1 << 24), "max_pages"));
  MLA_TRY(need_range(B, 1, (1 << 20), "B"));
  const long long cap = (long long)max_pages * MLA_PAGE;
  for (int b = 0; b < B; ++b) {
    const long long L = seqlens[b];
    if (L < 0 || L > cap) {
      if (bad_seq) *bad_seq = b;
      Check c;
      c.status = MLA_ERR_SHAPE;
      char buf[256];
      std::snprintf(buf, sizeof buf, "seqlens[%d] = %lld outside [0, %lld] (max_pages * 64)", b, L, cap);
      c.detail = buf;
      return c;
    }
    const long long n = (L + MLA_PAGE - 1) / MLA_PAGE;
    const int32_t* row = bt + (size_t)b * (size_t)max_pages;
    for (long long p = 0; p < n; ++p) {
      if (row[p] < 0 || row[p] >= num_pages) {
        if (bad_seq) *bad_seq = b;
        if (bad_page) *bad_page = (int)p;
        Check c;
        c.status = MLA_ERR_SHAPE;
        char buf[256];
        std::snprintf(buf, sizeof buf, "block_table[%d, %lld] = %d outside [0, %lld) (sequence of %lld tokens)", b,
                      p, (int)row[p], (long long)num_pages, L);
        c.detail = buf;
        return c;
      }
    }
  }
  return Check{};
}

inline size_t workspace_bytes(int B, int s_q, int H, int num_splits) {
  if (B < 1 || s_q < 1 || H < 1 || num_splits < 1) return 0;
  return (size_t)B * s_q * H * num_splits * (MLA_D_C + 1) * sizeof(float);
}

// ---- split planning -------------------------------------------------------
// mla_decode_paged concatenates the pages of all rows (b, i) in order and
// gives workgroup k of kScanGroups the page range [kW, (k+1)W). With
// num_splits S > 1 rows are cut at range borders and
//     W = max(ceil(P_tot / kScanGroups), ceil((n_max - 1) / (S - 1)), 1),
// which bounds any row to S pieces; with S = 1 rows are not cut, W is
// ceil(P_tot / kScanGroups) and a row goes whole to the range holding its
// middle page (first page + floor(n / 2)). The planner below evaluates that
// plan for every distinct W.
constexpr int kScanGroups = 256;

// Visible pages of every row (b, i), lengths clamped like the kernel does.
inline std::vector<int64_t> row_pages(const int32_t* seqlens, int B, int s_q, int max_pages) {
  std::vector<int64_t> n;
  n.reserve((size_t)B * s_q);
  const long long cap = (long long)max_pages * MLA_PAGE;
  for (int b = 0; b < B; ++b) {
    long long L = seqlens[b];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    for (int i = 0; i < s_q; ++i) {
      const long long v = L - s_q + i + 1;
      n.push_back(v > 0 ? (v + MLA_PAGE - 1) / MLA_PAGE : 0);
    }
  }
  return n;
}

// Time model of one scan, in units of ~0.105 us on MI355X: the slowest
// workgroup (2.8 us per page, ~10.5 us per row piece for its query loads,
// pipeline start and partial write), times the rounds needed when the GPU has
// fewer than kScanGroups CUs, plus writing and re-reading every partial.
inline long long scan_cost(const std::vector<int64_t>& n, int64_t W, bool cut, long long cus) {
  constexpr long long kPageCost = 27, kPieceCost = 100;
  long long pages[kScanGroups] = {}, pieces[kScanGroups] = {};
  long long total = 0;
  int64_t P = 0;
  for (const int64_t nr : n) {
    if (nr > 0) {
      if (cut) {
        const int64_t k0 = P / W, k1 = (P + nr - 1) / W;
        for (int64_t k = k0; k <= k1; ++k) {
          const int64_t a = P > k * W ? P : k * W;
          const int64_t e = P + nr < (k + 1) * W ? P + nr : (k + 1) * W;
          pages[k] += e - a;
          ++pieces[k];
        }
        total += k1 - k0 + 1;
      } else {
        const int64_t k = (P + nr / 2) / W;
        pages[k] += nr;
        ++pieces[k];
        ++total;
      }
    }
    P += nr;
  }
  long long span = 0;
  for (int k = 0; k < kScanGroups; ++k) {
    const long long t = kPageCost * pages[k] + kPieceCost * pieces[k];
    if (t > span) span = t;
  }
  const long long rounds = (kScanGroups + cus - 1) / cus;
  return span * rounds + total;
}

// Smallest S whose plan has the lowest modelled time.
inline int plan_rows(const std::vector<int64_t>& n, int max_pages, int num_cus) {
  const long long cus = num_cus > 0 ? num_cus : kScanGroups;
  int64_t p_tot = 0, n_max = 0;
  for (const int64_t nr : n) {
    p_tot += nr;
    if (nr > n_max) n_max = nr;
  }
  if (p_tot == 0) return 1;
  const int64_t w_base = (p_tot + kScanGroups - 1) / kScanGroups;
  int best_s = 1;
  long long best = scan_cost(n, w_base, false, cus);
  const int s_max = max_pages < 256 ? max_pages : 256;
  int64_t w_prev = -1;
  for (int S = 2; S <= s_max; ++S) {
    int64_t W = (n_max - 1 + S - 2) / (S - 1);
    if (W < w_base) W = w_base;
    if (W < 1) W = 1;
    if (W == w_prev) continue;  // the same plan with more slots
    w_prev = W;
    const long long c = scan_cost(n, W, true, cus);
    if (c < best) {
      best = c;
      best_s = S;
    }
  }
  return best_s;
}

// Split count for host-known lengths.
inline int plan_splits(const int32_t* seqlens, int B, int s_q, int max_pages, int num_cus) {
  if (seqlens == nullptr || B < 1 || s_q < 1 || max_pages < 1) return 1;
  if ((long long)B * s_q > (1LL << 22)) return 1;  // huge batches fill the GPU unsplit
  return plan_rows(row_pages(seqlens, B, s_q, max_pages), max_pages, num_cus);
}

// Split count when only the longest length is known: the plan for B
// sequences of max_len tokens and a block table just wide enough for them.
inline int recommended_splits(int B, int s_q, int max_len, int num_cus) {
  if (max_len < 1 || B < 1 || s_q < 1) return 1;
  const long long pages = ((long long)max_len + MLA_PAGE - 1) / MLA_PAGE;
  if (pages > (1 << 24)) return 1;
  std::vector<int32_t> lens((size_t)B, max_len);
  return plan_splits(lens.data(), B, s_q, (int)pages, num_cus);
}

}  // namespace mla
