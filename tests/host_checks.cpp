// Host-side argument checks, block-table validation and split planning of the
// MLA C ABI (mla_latent_kv_06_amd/csrc/validate.hpp), exercised without a GPU.
// tests/test_host_sanitized.py builds this with g++ under AddressSanitizer
// and UndefinedBehaviorSanitizer and runs it; any failed expectation or
// sanitizer report makes the process exit non-zero.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <vector>

#include "../mla_latent_kv_06_amd/csrc/validate.hpp"

static int g_fail = 0;

#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

static void* const A = reinterpret_cast<void*>(uintptr_t(1) << 20);   // aligned, never dereferenced
static void* const MIS = reinterpret_cast<void*>((uintptr_t(1) << 20) + 8);

static mla_status decode(const void* q_abs, const void* kv, int64_t num_pages, int max_pages, int B, int s_q, int H,
                         float scale, int S, const void* o_part) {
  return mla::check_decode(q_abs, A, kv, num_pages, A, max_pages, A, B, s_q, H, scale, S, o_part, A).status;
}

static void status_codes() {
  EXPECT(decode(A, A, 10, 4, 2, 1, 128, 0.07f, 2, A) == MLA_OK);
  EXPECT(decode(nullptr, A, 10, 4, 2, 1, 128, 0.07f, 2, A) == MLA_ERR_NULL);
  EXPECT(decode(A, MIS, 10, 4, 2, 1, 128, 0.07f, 2, A) == MLA_ERR_ALIGN);
  EXPECT(decode(A, A, 10, 4, 2, 1, 128, 0.07f, 2, MIS) == MLA_ERR_ALIGN);
  EXPECT(decode(A, A, 0, 4, 2, 1, 128, 0.07f, 2, A) == MLA_ERR_SHAPE);
  EXPECT(decode(A, A, 10, 0, 2, 1, 128, 0.07f, 1, A) == MLA_ERR_SHAPE);
  EXPECT(decode(A, A, 10, 4, 0, 1, 128, 0.07f, 2, A) == MLA_ERR_SHAPE);
  EXPECT(decode(A, A, 10, 4, 2, 0, 128, 0.07f, 2, A) == MLA_ERR_SHAPE);
  EXPECT(decode(A, A, 10, 4, 2, 4097, 128, 0.07f, 2, A) == MLA_ERR_SHAPE);
  EXPECT(decode(A, A, 10, 4, 2, 1, 64, 0.07f, 2, A) == MLA_ERR_SHAPE);
  EXPECT(decode(A, A, 10, 4, 2, 1, 128, 0.07f, 5, A) == MLA_ERR_SHAPE);
  EXPECT(decode(A, A, 10, 4, 2, 1, 128, 0.0f, 2, A) == MLA_ERR_SHAPE);
  EXPECT(decode(A, A, 10, 4, 2, 1, 128, -1.0f, 2, A) == MLA_ERR_SHAPE);
  EXPECT(decode(A, A, 10, 4, 2, 1, 128, std::numeric_limits<float>::quiet_NaN(), 2, A) == MLA_ERR_SHAPE);
  EXPECT(decode(A, A, 10, 4, 2, 1, 128, std::numeric_limits<float>::infinity(), 2, A) == MLA_ERR_SHAPE);
  // the plan's 32-bit page counts: B * s_q * max_pages must stay below 2^31
  EXPECT(decode(A, A, 10, 1 << 20, 1 << 12, 1, 128, 0.07f, 2, A) == MLA_ERR_SHAPE);
  EXPECT(mla::check_absorb(A, A, A, 1, 128).status == MLA_OK);
  EXPECT(mla::check_absorb(A, A, A, 0, 128).status == MLA_ERR_SHAPE);
  EXPECT(mla::check_absorb(A, MIS, A, 4, 128).status == MLA_ERR_ALIGN);
  EXPECT(mla::check_up_proj(A, A, nullptr, 4, 128).status == MLA_ERR_NULL);
  EXPECT(mla::check_combine(A, A, 1, 1, 128, 0, A, A).status == MLA_ERR_SHAPE);
  EXPECT(mla::check_combine_up(A, A, nullptr, 1, 1, 128, 2, A, A).status == MLA_ERR_NULL);
  EXPECT(mla::check_gather(A, 3, A, 1, A, 1, 0, A).status == MLA_ERR_SHAPE);
  EXPECT(mla::check_decompress(A, 3, A, 1, A, 1, 100, A, A, A, A).status == MLA_ERR_SHAPE);  // not a page multiple
  EXPECT(mla::check_rope_table(10000.0, 0, A, 1 << 22).status == MLA_ERR_SHAPE);
  EXPECT(mla::check_rope_table(-1.0, 8, A, 1 << 22).status == MLA_ERR_SHAPE);
  EXPECT(!mla::check_decode(nullptr, A, A, 10, A, 4, A, 2, 1, 128, 0.07f, 2, A, A).detail.empty());
}

static void static_scratch() {
  // the long workload (B = 16, 17 splits) fits; 64 splits do not
  const mla::ScratchLayout L = mla::scratch_layout(16, 1, 17);
  EXPECT(L.q_abs == 0 && L.o_part == (size_t)16 * 128 * 512 * 2);
  EXPECT(L.lse_part == L.o_part + (size_t)16 * 128 * 17 * 512 * 4);
  EXPECT(L.total % 256 == 0 && L.total <= mla::kStaticScratchBytes);
  auto st = [](int B, int s_q, int S, const void* out) {
    return mla::check_step_static(A, A, A, 10, A, 1024, A, B, s_q, 128, A, A, 0.07f, S, out, A).status;
  };
  EXPECT(st(16, 1, 17, A) == MLA_OK);
  EXPECT(st(16, 1, 64, A) == MLA_ERR_WORKSPACE);
  EXPECT(st(16, 1, 17, nullptr) == MLA_ERR_NULL);
  EXPECT(st(16, 1, 17, MIS) == MLA_ERR_ALIGN);
  EXPECT(st(1 << 20, 2, 1, A) == MLA_ERR_SHAPE);
}

static void block_tables() {
  const int32_t bt[2][4] = {{3, 0, -1, -1}, {1, 2, 4, -5}};
  int bs = 7, bp = 7;
  {
    const int32_t L[2] = {65, 130};
    EXPECT(mla::validate_block_table(&bt[0][0], 4, L, 2, 5, &bs, &bp).status == MLA_OK);
    EXPECT(bs == -1 && bp == -1);
    EXPECT(mla::validate_block_table(&bt[0][0], 4, L, 2, 4, &bs, &bp).status == MLA_ERR_SHAPE);
    EXPECT(bs == 1 && bp == 2);
  }
  {
    const int32_t L[2] = {129, 10};
    const mla::Check c = mla::validate_block_table(&bt[0][0], 4, L, 2, 5, &bs, &bp);
    EXPECT(c.status == MLA_ERR_SHAPE && bs == 0 && bp == 2 && !c.detail.empty());
  }
  {
    const int32_t L[2] = {65, 257};
    EXPECT(mla::validate_block_table(&bt[0][0], 4, L, 2, 5, &bs, &bp).status == MLA_ERR_SHAPE);
    EXPECT(bs == 1 && bp == -1);
    EXPECT(mla::validate_block_table(&bt[0][0], 4, L, 2, 5, nullptr, nullptr).status == MLA_ERR_SHAPE);
  }
  {
    const int32_t L[2] = {std::numeric_limits<int32_t>::min(), 0};
    EXPECT(mla::validate_block_table(&bt[0][0], 4, L, 2, 5, &bs, &bp).status == MLA_ERR_SHAPE);
    EXPECT(bs == 0 && bp == -1);
  }
  const int32_t L1[1] = {1};
  EXPECT(mla::validate_block_table(nullptr, 4, L1, 1, 5, &bs, &bp).status == MLA_ERR_NULL);
  EXPECT(mla::validate_block_table(&bt[0][0], 4, nullptr, 1, 5, &bs, &bp).status == MLA_ERR_NULL);
  EXPECT(mla::validate_block_table(&bt[0][0], 0, L1, 1, 5, &bs, &bp).status == MLA_ERR_SHAPE);
  // a large table checked end to end (heap-allocated, so ASan sees any overrun)
  const int B = 64, maxp = 512;
  std::vector<int32_t> big((size_t)B * maxp, -1), lens(B);
  for (int b = 0; b < B; ++b) {
    lens[b] = 1 + (b * 523) % (maxp * 64);
    for (int p = 0; p < (lens[b] + 63) / 64; ++p) big[(size_t)b * maxp + p] = (b * maxp + p) % 40000;
  }
  EXPECT(mla::validate_block_table(big.data(), maxp, lens.data(), B, 40000, &bs, &bp).status == MLA_OK);
  big[(size_t)(B - 1) * maxp + (lens[B - 1] - 1) / 64] = 40000;
  EXPECT(mla::validate_block_table(big.data(), maxp, lens.data(), B, 40000, &bs, &bp).status == MLA_ERR_SHAPE);
  EXPECT(bs == B - 1 && bp == (lens[B - 1] - 1) / 64);
}

static void planning() {
  EXPECT(mla::workspace_bytes(16, 1, 128, 17) == (size_t)16 * 128 * 17 * 513 * 4);
  EXPECT(mla::workspace_bytes(0, 1, 128, 17) == 0);
  EXPECT(mla::plan_splits(nullptr, 4, 1, 16, 256) == 1);
  std::vector<int32_t> uniform(16, 65536);
  const int s = mla::plan_splits(uniform.data(), 16, 1, 1024, 256);
  EXPECT(s >= 1 && s <= 256);
  std::vector<int32_t> ragged(64);
  for (int b = 0; b < 64; ++b) ragged[b] = 1 + (b * 7919) % 32768;
  const int r = mla::plan_splits(ragged.data(), 64, 1, 512, 256);
  EXPECT(r >= 1 && r <= 256);
  EXPECT(mla::recommended_splits(1, 1, 2048, 256) >= 1);
  EXPECT(mla::recommended_splits(1, 1, 0, 256) == 1);
  // lengths beyond the table are clamped, negative ones count as empty
  std::vector<int32_t> odd = {-5, 0, 1 << 30, 64};
  const int o = mla::plan_splits(odd.data(), 4, 3, 8, 256);
  EXPECT(o >= 1 && o <= 8);
}

int main() {
  status_codes();
  static_scratch();
  block_tables();
  planning();
  if (g_fail) {
    std::fprintf(stderr, "%d expectation(s) failed\n", g_fail);
    return 1;
  }
  std::printf("host checks ok\n");
  return 0;
}
