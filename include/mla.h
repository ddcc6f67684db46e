/*
 * mla.h -- C ABI of the absorbed Multi-Head Latent Attention (MLA) decode
 * library for AMD Instinct MI355X (gfx950).
 *
 * What is computed (MLA operator-teardown page, jh158.com, sections 1, 3, 4):
 *   per token and layer the cache holds a 512-wide latent c_KV followed by a
 *   64-wide decoupled RoPE key k_R (576 bf16 values). W_UK is absorbed into
 *   the query (q_abs = q_c . W_UK per head), so each score is
 *       s[h, t] = (q_abs[h] . c_KV[t] + q_R[h] . k_R[t]) / sqrt(128 + 64)
 *   and the latent output o_lat[h] = softmax(s[h]) . c_KV is up-projected
 *   per head through W_UV. The per-head 16384-wide keys never exist.
 * Long contexts are scanned in page-aligned splits whose partial results are
 *   merged by their log-sum-exp (stage 1 scan and stage 2 reduction of the
 *   MI355X Kimi K3 time-share study, jinnpan.com, "Inside the blocks").
 *
 * Sections below, in order: the absorbed path (absorb, split scan, merge,
 *   up-projection, and the merge fused with the up-projection); the cache
 *   append and RoPE; the decompressed branch for long chunks and its
 *   dispatch rule; the 8-bit (E4M3) and 4-bit (MXFP4) latent caches; the
 *   whole step in one launch; test aids.
 *
 * Conventions for every function below:
 *   - Pointers are DEVICE pointers unless stated otherwise, must be non-NULL
 *     and 16-byte aligned. Tensors are dense, row-major, innermost last.
 *   - bf16 is IEEE bfloat16 stored as uint16; fp32 is IEEE float.
 *   - The caller owns every buffer. The library allocates nothing, keeps no
 *     state besides cached device properties, and is safe to call from
 *     several host threads.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     with no host synchronisation. Results are valid once the caller has
 *     synchronised with that stream.
 *   - Arguments are validated on the host before any launch. A non-OK status
 *     means nothing was enqueued, except MLA_ERR_HIP, which reports a launch
 *     failure. Device faults surface at the caller's next synchronisation.
 *   - No C++ exception crosses this interface.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Problem constants (teardown page, section 3: 128 heads, content head dim
 * 128, latent 512, RoPE 64, page size 64). */
enum {
  MLA_HEADS = 128, /* attention heads H */
  MLA_D_HC = 128,  /* content dims per head of q_c, W_UK and W_UV rows */
  MLA_D_C = 512,   /* latent dims of c_KV */
  MLA_D_R = 64,    /* decoupled RoPE dims of q_R and k_R */
  MLA_ROW = 576,   /* bf16 values stored per token and layer */
  MLA_PAGE = 64    /* tokens per cache page */
};

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,      /* a required pointer is NULL */
  MLA_ERR_SHAPE = 2,     /* a size argument is out of range */
  MLA_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
  MLA_ERR_WORKSPACE = 4, /* a caller buffer is too small for the request */
  MLA_ERR_HIP = 5        /* the HIP runtime reported an error */
} mla_status;

/* Static, never-NULL name of a status code ("MLA_OK", ...). Unknown codes
 * give "MLA_ERR_UNKNOWN". */
const char* mla_status_string(int status);

/* Human-readable detail of the most recent non-OK status returned on the
 * calling host thread (which argument failed and why). Static per-thread
 * storage; never NULL; "" if nothing failed yet. */
const char* mla_last_error(void);

/* Absorb W_UK into the query (teardown page, section 4, absorbed path):
 *     q_abs[t, h, c] = sum_d q_c[t, h, d] * W_UK[h, d, c]
 * fp32 accumulation, result rounded to bf16 (round-to-nearest-even).
 *   q_c   bf16 [T, H, 128]   (T = batch * new tokens, any order)
 *   w_uk  bf16 [H, 128, 512] (the page's w_uk layout (nh, dhc, dc))
 *   q_abs bf16 [T, H, 512]   output
 *   T >= 1, H == MLA_HEADS. */
mla_status mla_absorb_q(const void* q_c, const void* w_uk, void* q_abs,
                        int64_t T, int H, void* stream);

/* Bytes of o_part plus lse_part for mla_decode_paged with these sizes
 * (B * s_q * H * num_splits * (512 + 1) * 4). Host-only, no validation;
 * returns 0 for non-positive arguments. */
size_t mla_decode_workspace_bytes(int B, int s_q, int H, int num_splits);

/* A split count for mla_decode_paged (host-only heuristic; max_len is the
 * longest sequence in tokens, num_cus the GPU's compute units, 256 if <= 0):
 * mla_plan_splits for B sequences of max_len tokens and a block table just
 * wide enough for them. The result is in [1, min(ceil(max_len / 64), 256)]
 * (1 if max_len < 1). */
int mla_recommended_splits(int B, int s_q, int max_len, int num_cus);

/* Split count for a batch whose lengths are known on the host
 * (seqlens_host: HOST pointer to B int32 lengths, clamped as
 * mla_decode_paged clamps them): the smallest S whose scan plan minimises a
 * time model of the launch (the slowest workgroup's pages and row pieces,
 * plus writing and re-reading every partial). Returns 1 for NULL or
 * non-positive sizes and for B * s_q above 2^22; otherwise a value in
 * [1, min(max_pages, 256)]. */
int mla_plan_splits(const int32_t* seqlens_host, int B, int s_q, int max_pages, int num_cus);

/* HOST function (test and debug aid): check a block table and its lengths
 * against the contract of mla_decode_paged and the other paged calls, which
 * do not check it on the device (they clamp every entry into the cache, so a
 * bad entry reads another page's rows instead of faulting; the teardown page,
 * section 5, lists such address faults among the gather's failure modes).
 *   block_table int32 [B, max_pages], seqlens int32 [B]: HOST pointers
 *   bad_seq, bad_page: HOST pointers (either may be NULL) that receive the
 *     first offending sequence and logical page in (b, p) order; page -1
 *     when the sequence's length is out of range; both -1 if all is valid
 * Returns MLA_OK when every length lies in [0, max_pages * 64] and every
 * entry a decode reads (logical pages p < ceil(L_b / 64)) lies in
 * [0, num_pages); MLA_ERR_SHAPE otherwise (mla_last_error() names the entry);
 * MLA_ERR_NULL for a NULL table or length array; MLA_ERR_SHAPE for
 * B, max_pages or num_pages out of the ranges mla_decode_paged accepts.
 * Entries past a sequence's pages are not examined. Reads only. */
mla_status mla_validate_block_table(const int32_t* block_table, int max_pages, const int32_t* seqlens, int B,
                                    int64_t num_pages, int* bad_seq, int* bad_page);

/* Debug switch (environment variable, read at every call): with
 * MLA_DEBUG_CHECKS set to anything but "" or "0", mla_decode_paged, its 8-bit
 * and 4-bit forms and mla_decode_step* copy block_table and seqlens from the
 * device after the caller's stream has drained, run the check above on them,
 * and return its status (mla_last_error() prefixed "MLA_DEBUG_CHECKS:")
 * without launching when the table is bad. The copy allocates host memory and
 * synchronises the stream, so the switch is for debugging only and must stay
 * off under graph capture; mla_decode_step_static never applies it. */

/* Stage 1: split scan of the paged latent cache, absorbed scores, online
 * softmax, P . c_KV on matrix cores (teardown page, section 4 absorbed
 * scores; K3 study "Inside the blocks" stage 1).
 *   q_abs       bf16 [B, s_q, H, 512]   absorbed queries
 *   q_r         bf16 [B, s_q, H, 64]    rotated RoPE queries
 *   kv_cache    bf16 [num_pages, 64, 576]; row = c_KV (0..511), k_R (512..575)
 *   block_table int32 [B, max_pages]: logical page p of sequence b lives in
 *               physical page block_table[b, p]. Only the first
 *               ceil(L_b / 64) entries are read; they must lie in
 *               [0, num_pages). Others (e.g. -1) are never read. Entries out
 *               of range are clamped into [0, num_pages) so no access leaves
 *               the cache; the affected rows' results are then unspecified.
 *   seqlens     int32 [B]: L_b = tokens in the cache for sequence b,
 *               including the s_q new ones. Values are clamped to
 *               [0, max_pages * 64].
 *   softmax_scale  multiplies q_abs.c_KV + q_R.k_R (1/sqrt(192) for DeepSeek);
 *               must be positive and finite.
 *   num_splits  S in [1, max_pages]: the partial slots per row. Query i of
 *               sequence b sees tokens t <= L_b - s_q + i, i.e. row (b, i)
 *               has n = ceil((L_b - s_q + i + 1) / 64) pages. The scan
 *               concatenates the pages of all rows in (b, i) order (P_tot in
 *               all, row r starting at page P_r) and gives each of 256
 *               workgroups an equal range of W pages, so ragged batches are
 *               balanced:
 *                 S > 1: W = max(ceil(P_tot / 256), ceil((n_max - 1)/(S - 1)), 1);
 *                        the piece of row r inside range k (pages
 *                        [kW, (k+1)W)) goes to slot k - floor(P_r / W);
 *                 S = 1: W = ceil(P_tot / 256); rows are not cut, each goes
 *                        to slot 0.
 *               Slots a row does not use are empty. The plan depends on the
 *               lengths of the whole batch (not on any other input); see
 *               mla_plan_splits for choosing S. B * s_q * max_pages must be
 *               below 2^31.
 *   o_part      fp32 [B, s_q, H, num_splits, 512] output: each non-empty
 *               split's softmax-normalised latent output; the rows of an
 *               empty split are not written
 *   lse_part    fp32 [B, s_q, H, num_splits] output: natural-log
 *               log-sum-exp of the split's scaled scores (-inf if empty)
 * B >= 1, 1 <= s_q <= 4096, H == MLA_HEADS, 1 <= max_pages,
 * num_pages >= 1. */
mla_status mla_decode_paged(const void* q_abs, const void* q_r,
                            const void* kv_cache, int64_t num_pages,
                            const int32_t* block_table, int max_pages,
                            const int32_t* seqlens, int B, int s_q, int H,
                            float softmax_scale, int num_splits,
                            float* o_part, float* lse_part, void* stream);

/* Stage 2: merge split partials by their log-sum-exp (K3 study, "Inside the
 * blocks", KV-split reduction):
 *     LSE = M + ln sum_s exp(lse_s - M),  M = max_s lse_s
 *     o   = sum_s exp(lse_s - LSE) * o_s
 * A split with lse_s = -inf is empty: its o_part row is never read (it may
 * hold anything). A row whose splits are all empty gives o = 0 and
 * LSE = -inf.
 *   o_part   fp32 [B, s_q, H, num_splits, 512], lse_part fp32 [B, s_q, H, num_splits]
 *   o_lat    fp32 [B, s_q, H, 512] output,  lse fp32 [B, s_q, H] output
 * B >= 1, s_q >= 1, H == MLA_HEADS, num_splits >= 1. */
mla_status mla_combine_splits(const float* o_part, const float* lse_part,
                              int B, int s_q, int H, int num_splits,
                              float* o_lat, float* lse, void* stream);

/* Stage 2 fused with the up-projection: merges the split partials exactly as
 * mla_combine_splits does and up-projects each merged row as mla_up_proj
 * does, in one pass that never writes o_lat (one read of o_part and W_UV).
 *   o_part, lse_part  as for mla_combine_splits (empty splits never read)
 *   w_uv   bf16 [H, 128, 512]
 *   out    bf16 [B * s_q, H, 128] output (rows in (b, i) order)
 *   lse    fp32 [B, s_q, H] output, as mla_combine_splits
 * B >= 1, s_q >= 1, H == MLA_HEADS, num_splits >= 1. */
mla_status mla_combine_up_proj(const float* o_part, const float* lse_part, const void* w_uv, int B, int s_q,
                               int H, int num_splits, void* out, float* lse, void* stream);

/* Per-head up-projection of the latent output (W_UV has W_UK's layout):
 *     out[t, h, d] = sum_c o_lat[t, h, c] * W_UV[h, d, c]
 * o_lat is split into a bf16 high part and a bf16 remainder so the fp32
 * input keeps ~16 significant bits on bf16 matrix cores; fp32 accumulation;
 * result rounded to bf16.
 *   o_lat fp32 [T, H, 512], w_uv bf16 [H, 128, 512], out bf16 [T, H, 128]
 *   T >= 1, H == MLA_HEADS. */
mla_status mla_up_proj(const float* o_lat, const void* w_uv, void* out,
                       int64_t T, int H, void* stream);

/* ---- the step before the decode path: cache append and RoPE -------------
 * The decoupled RoPE parts are rotated in fp32 from an fp32 table with fp32
 * multiply-adds (teardown page: RoPE compute type fp32, section 3; an fp32
 * table and fp32 multiply-adds against the phase error of fp16, section 4).
 * Pair j of a 64-value vector x is (x[2j], x[2j+1]); at position p it turns
 * counter-clockwise by p * theta_j, theta_j = base^(-2j/64):
 *     y[2j]   = x[2j] cos - x[2j+1] sin,   y[2j+1] = x[2j] sin + x[2j+1] cos
 * computed as fp32 fma and rounded once to bf16. Token i of an s_q-token
 * chunk of sequence b has position L_b - s_q + i, where seqlens[b] = L_b
 * already counts the chunk (the same rule as the causal limit of
 * mla_decode_paged). */

/* HOST function: fill the rotation table for positions 0 .. max_pos-1,
 *     table[(p * 32 + j) * 2 + 0] = cos(p * theta_j),  [... + 1] = sin(...)
 * computed in double and rounded to float. `table` is a HOST pointer to
 * max_pos * 64 floats (no alignment rule); copy it to the device for the two
 * functions below. base > 0 and finite; 1 <= max_pos <= 2^22.
 * Returns MLA_ERR_NULL / MLA_ERR_SHAPE on bad arguments. */
mla_status mla_rope_table(double base, int max_pos, float* table);

/* Write a chunk of new tokens into the paged cache:
 *     cache row L_b - s_q + i of sequence b  <-  c_new[b, i] ++ rope(kr_new[b, i])
 * i.e. physical page block_table[b, p / 64], row p % 64 with p the token's
 * position; the 512 c_KV values are copied bit for bit, the 64 k_R values
 * rotated by p. Tokens with p < 0 or p >= min(max_pages * 64, max_pos) are
 * not written. Other rows of the cache are not touched.
 *   c_new    bf16 [B, s_q, 512]
 *   kr_new   bf16 [B, s_q, 64]   (k_R before rotation)
 *   rope     fp32 [max_pos, 32, 2] table from mla_rope_table (device copy)
 *   kv_cache bf16 [num_pages, 64, 576], updated in place
 *   block_table, seqlens: as mla_decode_paged (entries are clamped into
 *   [0, num_pages), so a bad entry cannot write outside the cache)
 * B >= 1, 1 <= s_q <= 4096, B * s_q <= 2^24, num_pages >= 1,
 * max_pages >= 1, max_pos >= 1. Two tokens that map to the same cache row
 * (a block table that shares pages between sequences) race. */
mla_status mla_append_latent(const void* c_new, const void* kr_new, const float* rope, int max_pos,
                             void* kv_cache, int64_t num_pages, const int32_t* block_table, int max_pages,
                             const int32_t* seqlens, int B, int s_q, void* stream);

/* Rotate the decoupled RoPE part of the chunk's queries in place:
 *     q_r[b, i, h, :] <- rope(q_r[b, i, h, :]) at position L_b - s_q + i
 * Rows whose position is negative or >= max_pos are left unchanged.
 *   q_r  bf16 [B, s_q, H, 64], in place
 *   rope fp32 [max_pos, 32, 2] (device copy of mla_rope_table's table)
 * B >= 1, 1 <= s_q <= 4096, H == MLA_HEADS, B * s_q <= 2^21, max_pos >= 1. */
mla_status mla_rope_q(void* q_r, const float* rope, int max_pos, const int32_t* seqlens, int B, int s_q, int H,
                      void* stream);

/* ---- decompressed branch for long chunks ---------------------------------
 * The teardown page keeps the absorbed form for chunks of up to 256 new
 * tokens (section 3: kPrefillThresh and the plugin's
 * prefill_absorption_threshold) and decompresses the latent cache per head
 * above that (path A of section 4), in two stages:
 *   K[b, h, t, :] = W_UK[h] . c_KV[t],  V[b, h, t, :] = W_UV[h] . c_KV[t]
 *   out[b, i, h] = softmax_t((q_c[b,i,h] . K[b,h,t] + q_R[b,i,h] . k_R[t]) * scale) . V[b,h,t]
 * over t <= L_b - s_q + i (the causal rule of mla_decode_paged); out is the
 * final per-head output (no up-projection). */

/* 1 if an s_q-token chunk takes the absorbed path (s_q <= 256), else 0. */
int mla_prefill_uses_absorption(int s_q);

/* Bytes of one of the K and V buffers: B * 128 * max_len * 128 16-bit values
 * (0 for non-positive sizes). */
size_t mla_decompressed_kv_bytes(int B, int max_len);

/* Stage 1: per-head keys and values of every cached token, bf16 MFMA with
 * fp32 accumulation, rounded once: keys to bf16, values to fp16 (the
 * attention's P.V product runs in fp16, three more significant bits than
 * bf16; values must stay below 65504 in magnitude, which the method's
 * weight scale keeps them far from).
 *   kv_cache, block_table, seqlens, num_pages, max_pages: as mla_decode_paged
 *   w_uk, w_uv  bf16 [H, 128, 512]
 *   k_nope      bf16 [B, H, max_len, 128] output (head-major)
 *   v           fp16 [B, H, max_len, 128] output (head-major)
 *   rows t < min(L_b, max_len) are written, rows from there to the end of
 *   that 64-token page are zero-filled, later rows are not touched
 * B >= 1, max_len >= 1 and a multiple of 64 (MLA_PAGE), B * max_len <= 2^31. */
mla_status mla_decompress_kv(const void* kv_cache, int64_t num_pages, const int32_t* block_table, int max_pages,
                             const int32_t* seqlens, int B, int max_len, const void* w_uk, const void* w_uv,
                             void* k_nope, void* v, void* stream);

/* Stage 2: causal attention over stage 1's K and V and the cache's k_R.
 *   q_c bf16 [B, s_q, H, 128], q_r bf16 [B, s_q, H, 64] (rotated)
 *   k_nope, v  from mla_decompress_kv with the same max_len and inputs
 *              (the attention reads whole pages of K and V; the zero-filled
 *              page tails keep garbage out of P . V)
 *   out bf16 [B, s_q, H, 128], lse fp32 [B, s_q, H] (natural log of the
 *   sum of exp(scaled score)); a query with no visible key gets out = 0 and
 *   lse = -inf. Queries see at most min(L_b, max_len) keys.
 * B >= 1, s_q >= 1, B * s_q <= 2^24, H == MLA_HEADS, max_len as above,
 * softmax_scale positive and finite. */
mla_status mla_prefill_mha(const void* q_c, const void* q_r, const void* k_nope, const void* v, int max_len,
                           const void* kv_cache, int64_t num_pages, const int32_t* block_table, int max_pages,
                           const int32_t* seqlens, int B, int s_q, int H, float softmax_scale, void* out, float* lse,
                           void* stream);

/* ---- 8-bit latent cache ---------------------------------------------------
 * The teardown page reads a quantized latent cache with 16-byte vector loads
 * that need 16-byte aligned page bases and dimension offsets (section 5). This
 * library's 8-bit cache stores c_KV in OCP FP8 E4M3 (1 sign, 4 exponent bits
 * with bias 7, 3 mantissa bits; largest finite value 448; no infinities) with
 * one power-of-two scale per token, and keeps k_R in bf16:
 *   scale 2^k, k the smallest integer with max_c |c_KV[c]| <= 448 * 2^k,
 *     clamped to [-126, 127] (an all-zero row gets 2^-126), so nothing saturates;
 *   code[c] = c_KV[c] / 2^k rounded to the nearest E4M3 value, ties to even,
 *     with the sign of c_KV[c] (a negative value that rounds to 0 becomes -0);
 *   stored value = E4M3(code[c]) * 2^k.
 * A page of 64 tokens is MLA_FP8_PAGE_BYTES = 41216 bytes, three arrays:
 *   bytes [0, 32768)      uint8 codes [64][512]
 *   bytes [32768, 40960)  bf16 k_R [64][64]
 *   bytes [40960, 41216)  fp32 scales [64] (each exactly 2^k)
 * The cache holds 644 bytes per token instead of 1152. Decoding over it gives
 * the attention of mla_decode_paged over the stored values (the scan converts
 * codes to bf16 exactly and computes as the bf16 scan does). c_KV inputs must
 * be finite. */
enum { MLA_FP8_PAGE_BYTES = 41216 };

/* Convert a bf16 cache to the 8-bit layout page for page (page p of kv_fp8
 * holds the 64 rows of page p of kv_cache).
 *   kv_cache bf16 [num_pages, 64, 576];  kv_fp8 uint8 [num_pages, 41216] output
 * 1 <= num_pages <= 2^26. */
mla_status mla_quantize_cache_fp8(const void* kv_cache, int64_t num_pages, void* kv_fp8, void* stream);

/* mla_append_latent into the 8-bit cache: c_new[b, i] quantized as above
 * (one scale per token), kr_new[b, i] rotated in fp32 and rounded to bf16.
 * kv_fp8 uint8 [num_pages, 41216], updated in place; all other arguments and
 * rules as mla_append_latent. */
mla_status mla_append_latent_fp8(const void* c_new, const void* kr_new, const float* rope, int max_pos,
                                 void* kv_fp8, int64_t num_pages, const int32_t* block_table, int max_pages,
                                 const int32_t* seqlens, int B, int s_q, void* stream);

/* mla_decode_paged over the 8-bit cache: kv_fp8 uint8 [num_pages, 41216];
 * every other argument, rule and output as mla_decode_paged (feed o_part and
 * lse_part to mla_combine_splits or mla_combine_up_proj). */
mla_status mla_decode_paged_fp8(const void* q_abs, const void* q_r,
                                const void* kv_fp8, int64_t num_pages,
                                const int32_t* block_table, int max_pages,
                                const int32_t* seqlens, int B, int s_q, int H,
                                float softmax_scale, int num_splits,
                                float* o_part, float* lse_part, void* stream);

/* ---- 4-bit latent cache ---------------------------------------------------
 * The teardown page's quantized gather is of a 4-bit (NVFP4) cache (section
 * 5). This library's 4-bit cache is the OCP microscaling form that the gfx950
 * matrix cores read directly, MXFP4: c_KV as E2M1 elements (1 sign, 2
 * exponent bits with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2,
 * 3, 4, 6; no infinities or NaN) with one E8M0 scale per 32 consecutive dims
 * of a token (16 per row), and k_R kept in bf16:
 *   block scale 2^k, k the smallest integer with max over the block of
 *     |c_KV[c]| <= 6 * 2^k, clamped to [-126, 127] (a zero block gets 2^-126),
 *     so nothing saturates; stored as the byte k + 127;
 *   code[c] = c_KV[c] / 2^k rounded to the nearest E2M1 value, ties to the
 *     even code, with the sign of c_KV[c] (a negative value that rounds to 0
 *     becomes -0); two codes per byte, the even dim in the low nibble;
 *   stored value = E2M1(code[c]) * 2^k.
 * A page of 64 tokens is MLA_MXFP4_PAGE_BYTES = 25600 bytes, three arrays:
 *   bytes [0, 16384)      uint8 codes [64][256]  (block u of a row = bytes 16u .. 16u+15)
 *   bytes [16384, 24576)  bf16 k_R [64][64]
 *   bytes [24576, 25600)  uint8 scales [64][16] (E8M0, k + 127)
 * The cache holds 400 bytes per token instead of 1152. Decoding over it gives
 * the attention of mla_decode_paged over the stored values: scores on the
 * block-scaled matrix-core instruction straight from the codes (the query as
 * two E4M3 terms, exact except for values under 2^-13 of their 32-dim block's
 * largest), V dequantized to bf16 exactly. Scale bytes 0 and 255 never occur
 * in pages this library writes and are not valid input. c_KV inputs must be
 * finite. */
enum { MLA_MXFP4_PAGE_BYTES = 25600 };

/* Convert a bf16 cache to the 4-bit layout page for page (page p of kv_fp4
 * holds the 64 rows of page p of kv_cache).
 *   kv_cache bf16 [num_pages, 64, 576];  kv_fp4 uint8 [num_pages, 25600] output
 * 1 <= num_pages <= 2^26. */
mla_status mla_quantize_cache_mxfp4(const void* kv_cache, int64_t num_pages, void* kv_fp4, void* stream);

/* mla_append_latent into the 4-bit cache: c_new[b, i] quantized as above
 * (one scale per 32-dim block), kr_new[b, i] rotated in fp32 and rounded to
 * bf16. kv_fp4 uint8 [num_pages, 25600], updated in place; all other
 * arguments and rules as mla_append_latent. */
mla_status mla_append_latent_mxfp4(const void* c_new, const void* kr_new, const float* rope, int max_pos,
                                   void* kv_fp4, int64_t num_pages, const int32_t* block_table, int max_pages,
                                   const int32_t* seqlens, int B, int s_q, void* stream);

/* mla_decode_paged over the 4-bit cache: kv_fp4 uint8 [num_pages, 25600];
 * every other argument, rule and output as mla_decode_paged (feed o_part and
 * lse_part to mla_combine_splits or mla_combine_up_proj). */
mla_status mla_decode_paged_mxfp4(const void* q_abs, const void* q_r,
                                  const void* kv_fp4, int64_t num_pages,
                                  const int32_t* block_table, int max_pages,
                                  const int32_t* seqlens, int B, int s_q, int H,
                                  float softmax_scale, int num_splits,
                                  float* o_part, float* lse_part, void* stream);

/* ---- the whole step in one launch ---------------------------------------
 * mla_absorb_q -> mla_decode_paged -> mla_combine_splits -> mla_up_proj as the
 * four phases of one cooperative kernel (256 workgroups, one per CU, separated
 * by grid-wide barriers), for short contexts where the step is a chain of
 * small dependent kernels. Results are bit-identical to that sequence of
 * calls with the same arguments: q_abs, o_part/lse_part, o_lat/lse and out are
 * all written.
 *   q_c bf16 [B, s_q, H, 128], q_r bf16 [B, s_q, H, 64] (rotated)
 *   kv_cache, num_pages, block_table, max_pages, seqlens, softmax_scale,
 *       num_splits: as mla_decode_paged
 *   w_uk, w_uv bf16 [H, 128, 512]
 *   q_abs bf16 [B, s_q, H, 512], o_part fp32 [B, s_q, H, num_splits, 512],
 *   lse_part fp32 [B, s_q, H, num_splits], o_lat fp32 [B, s_q, H, 512]:
 *       caller-owned intermediates (written)
 *   out bf16 [B, s_q, H, 128], lse fp32 [B, s_q, H]: the step's outputs
 * Argument rules as mla_decode_paged, and B * s_q <= 2^20. Returns MLA_ERR_HIP
 * if the device cannot hold all 256 workgroups at once (the launch is refused,
 * nothing runs). */
mla_status mla_decode_step(const void* q_c, const void* q_r, const void* kv_cache, int64_t num_pages,
                           const int32_t* block_table, int max_pages, const int32_t* seqlens, int B, int s_q,
                           int H, const void* w_uk, const void* w_uv, float softmax_scale, int num_splits,
                           void* q_abs, float* o_part, float* lse_part, float* o_lat, void* out, float* lse,
                           void* stream);

/* mla_decode_step over the 8-bit cache (kv_fp8 uint8 [num_pages, 41216]);
 * bit-identical to mla_absorb_q -> mla_decode_paged_fp8 -> mla_combine_splits
 * -> mla_up_proj. */
mla_status mla_decode_step_fp8(const void* q_c, const void* q_r, const void* kv_fp8, int64_t num_pages,
                               const int32_t* block_table, int max_pages, const int32_t* seqlens, int B, int s_q,
                               int H, const void* w_uk, const void* w_uv, float softmax_scale, int num_splits,
                               void* q_abs, float* o_part, float* lse_part, float* o_lat, void* out, float* lse,
                               void* stream);

/* mla_decode_step over the 4-bit cache (kv_fp4 uint8 [num_pages, 25600]);
 * bit-identical to mla_absorb_q -> mla_decode_paged_mxfp4 -> mla_combine_splits
 * -> mla_up_proj. */
mla_status mla_decode_step_mxfp4(const void* q_c, const void* q_r, const void* kv_fp4, int64_t num_pages,
                                 const int32_t* block_table, int max_pages, const int32_t* seqlens, int B, int s_q,
                                 int H, const void* w_uk, const void* w_uv, float softmax_scale, int num_splits,
                                 void* q_abs, float* o_part, float* lse_part, float* o_lat, void* out, float* lse,
                                 void* stream);

/* ---- the step without caller workspace -----------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 * mla_decode_step_static computes what mla_decode_step computes (out and lse)
 * without the caller-owned intermediates: q_abs and the split partials live in
 * one static device array of MLA_STATIC_SCRATCH_BYTES (96 MiB), which the
 * library holds on every GPU it runs on until the process ends. It launches
 * mla_absorb_q -> mla_decode_paged -> mla_combine_up_proj (the fast kernels of
 * the step, not the cooperative one), so out and lse equal those three calls
 * bit for bit, and meet mla_decode_step's within rounding of the fused merge.
 * It allocates nothing (no hipMalloc, hipFree or allocating library call).
 *   q_c, q_r, kv_cache, num_pages, block_table, max_pages, seqlens, B, s_q, H,
 *   w_uk, w_uv, softmax_scale, num_splits: as mla_decode_step
 *   out bf16 [B * s_q, H, 128], lse fp32 [B, s_q, H]: outputs
 * Needs the scratch layout q_abs [B*s_q, H, 512] bf16, o_part
 * [B*s_q, H, num_splits, 512] fp32 and lse_part [B*s_q, H, num_splits] fp32,
 * each rounded up to 256 bytes, to fit in the array: otherwise
 * MLA_ERR_WORKSPACE and nothing is enqueued (B = 16, num_splits = 17 needs
 * about 70 MiB). `stream` must belong to the current device (MLA_ERR_HIP
 * otherwise). Calls on one GPU share its array: two calls whose executions
 * overlap on that GPU (different streams, or host threads) race and give
 * undefined results; calls ordered on one stream are safe. The array keeps
 * the last call's contents; nothing in it needs clearing between calls. */
enum { MLA_STATIC_SCRATCH_BYTES = 96 * 1024 * 1024 };
mla_status mla_decode_step_static(const void* q_c, const void* q_r, const void* kv_cache, int64_t num_pages,
                                  const int32_t* block_table, int max_pages, const int32_t* seqlens, int B, int s_q,
                                  int H, const void* w_uk, const void* w_uv, float softmax_scale, int num_splits,
                                  void* out, float* lse, void* stream);

/* Test and debug aid: gather the logical cache rows of each sequence through
 * the block table with the same address arithmetic as mla_decode_paged.
 *   out bf16 [B, max_len, 576]: row t of sequence b is the cache row of token
 *   t for t < min(L_b, max_len) and zero otherwise.
 * Same argument rules as mla_decode_paged; max_len >= 1. */
mla_status mla_debug_gather(const void* kv_cache, int64_t num_pages,
                            const int32_t* block_table, int max_pages,
                            const int32_t* seqlens, int B, int max_len,
                            void* out, void* stream);

/* Measurement aids for reports that set a kernel's roofline fractions (taken
 * against the published peaks) beside what this board achieves with nothing
 * else to do; not part of the decode path. Both enqueue one kernel on
 * `stream` and write to `sink` (device, 16-byte aligned, at least
 * MLA_BENCH_SINK_FLOATS floats) only values of no meaning, which keep the work
 * from being optimised away. MLA_ERR_NULL / MLA_ERR_ALIGN / MLA_ERR_SHAPE as
 * for the other calls.
 *
 * mla_bench_stream_read: reads each 16-byte chunk of buf (device, 16-byte
 * aligned, `bytes` a positive multiple of 16) once, with non-temporal vector
 * loads (the scan's cache policy), from 2048 workgroups of 256 threads: the
 * achievable streaming-read rate is bytes / duration.
 *
 * mla_bench_mfma: 256 workgroups of 4 waves (one wave per SIMD, the scan's
 * launch shape); each wave runs `iters` (>= 1) rounds of four independent
 * chains of v_mfma_f32_32x32x16_bf16 on register-resident pseudo-random bf16
 * operands, i.e. 256 * 4 * 4 * iters * 32768 FLOP with no memory traffic: the
 * sustained dense bf16 matrix rate is that over the duration. */
enum { MLA_BENCH_SINK_FLOATS = 4096 };
mla_status mla_bench_stream_read(const void* buf, int64_t bytes, float* sink, void* stream);
mla_status mla_bench_mfma(int64_t iters, float* sink, void* stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* MLA_H */
