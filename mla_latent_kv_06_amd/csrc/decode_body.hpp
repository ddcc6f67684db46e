// Stage 1 of absorbed MLA decode: split scan of the paged latent cache.
//
// One workgroup = one (sequence b, query i, split s) work item and all 128
// heads, so every 1152-byte cache row is fetched from HBM once per work item
// and shared by all heads through LDS (absorbed scores of the MLA
// operator-teardown page, section 4; split scan of the K3 time-share study,
// "Inside the blocks").
//
// Work split inside the workgroup (4 waves, one per SIMD):
//   * QK: wave w owns heads 32w..32w+31. S^T = K . Q^T on
//     v_mfma_f32_32x32x16_bf16 with A = 32 cache rows x 16 dims read from LDS
//     and B = the wave's queries, held in 144 VGPRs for all 576 dims. A lane
//     ends up owning one head and 16 of the tile's 32 tokens.
//   * softmax in the exp2 domain against a per-head reference max taken from
//     the split's first tile; P = exp2(x - ref) may grow to 2^64, which bf16
//     and the fp32 accumulators hold without loss, so the accumulator is
//     never rescaled. Each lane also tracks the true running max; if any
//     score exceeded its reference by more than 64, the workgroup rescans
//     the split once with the exact max as reference.
//   * PV: wave w owns latent columns 128w..128w+127 for ALL heads. Every
//     wave publishes its P^T tile (bf16, already in MFMA operand layout) to
//     LDS, and each wave reads V^T only for its own columns with
//     ds_read_b64_tr_b16. This reads each V element from LDS once instead of
//     once per head group (transposed reads run at about half the rate of
//     plain 16-byte reads).
//   * software pipeline: iteration i runs QK(i), then softmax(i) interleaved
//     with PV(i-1), so the softmax VALU work overlaps matrix-core work and
//     P(i) is published in a double-buffered slot that the next iteration's
//     barrier makes visible. The last quarter of PV(i-1) waits until after
//     the next barrier, where its MFMAs hide the latency of the first K reads,
//     and the first PV(i-1) operands are read during the last QK(i) MFMAs.
//   * the cache streams through a ring of 4 LDS stages of 32 tokens (36 KiB,
//     half a page) filled with 16-byte direct-to-LDS loads; while one stage
//     is read by QK and one by PV, the next tile is landing and the one after
//     is issued, spread between the QK MFMAs.
//   * LDS rows are 72 chunks of 16 bytes; the low 3 bits of a chunk index are
//     XOR-swizzled with ((t&3)<<1) ^ ((t>>2)&7) of the row t, which keeps the
//     16-byte row reads of QK and the transposed 8-byte reads of PV free of
//     bank conflicts.
#pragma once

#include <type_traits>

#include "mla_device.hpp"
#include "decode.hpp"
#include "fp8_cache.hpp"
#include "mxfp4_cache.hpp"

namespace mla {

namespace {

constexpr int kTok = 32;                          // tokens per LDS stage
constexpr int kStages = 4;                        // LDS ring depth
constexpr int kStageBytes = kTok * kRowBytes;     // 36864
constexpr int kThreads = 256;
constexpr int kDmaPerThread = kStageBytes / (kThreads * 16);  // 9
constexpr int kPBytes = 2 * 4 * 2 * 1024;         // [slot][wave][k-step][64 lanes x 16 B]
constexpr int kLdsBytes = kStages * kStageBytes + kPBytes;   // 163840 = all of it
constexpr float kRefSlack = 64.0f;                // log2 headroom above the reference max
constexpr int kScanGroups = 256;                  // workgroups of a scan (one per MI355X CU)
#ifndef MLA_DMA_GAP
#define MLA_DMA_GAP 4
#endif
constexpr int kDmaGap = MLA_DMA_GAP;              // QK MFMAs between two of the next tile's loads (bf16)
static_assert(kDmaPerThread * kThreads * 16 == kStageBytes, "stage must split into 16-byte loads");
static_assert(kLdsBytes <= 163840, "LDS budget");

// 8-bit cache: a stage holds the tile's 32 rows of 512 codes, then its 32 k_R
// rows of 128 bytes, then its 32 scales; a thread issues 6 loads per tile
// (4 code chunks, 1 k_R chunk, and in lanes 0-1 of every wave 1 scale chunk).
constexpr int kStage8Rope = kTok * kDc;                      // 16384
constexpr int kStage8Scale = kStage8Rope + kTok * kDr * 2;   // 20480
constexpr int kStage8Bytes = kStage8Scale + kTok * 4;        // 20608
constexpr int kDma8PerThread = 6;
static_assert(4 * kThreads * 16 == kStage8Rope && kThreads * 16 == kTok * kDr * 2 && 8 * 16 == kTok * 4,
              "8-bit stage must split into 16-byte loads");
static_assert(kStage8Bytes % 16 == 0, "8-bit stages start on 16-byte boundaries");

// 4-bit cache: a stage holds the tile's 32 rows of 256 code bytes (16-byte
// chunk u of a row = MX block u, at chunk slot u ^ (row & 7)), then its 32 k_R
// rows, then its 32 rows of 16 scale bytes; a thread issues 4 loads per tile
// (2 code chunks, 1 k_R chunk, and in lanes 0-7 of every wave 1 scale chunk).
// V is dequantized once per tile into one of two bf16 tiles in the bf16
// stage layout, which PV reads as in the bf16 scan.
constexpr int kStage4Rope = kTok * kFp4RowBytes;             // 8192
constexpr int kStage4Scale = kStage4Rope + kTok * kDr * 2;   // 12288
constexpr int kStage4Bytes = kStage4Scale + kTok * (kDc / kMxBlock);  // 12800
constexpr int kDma4PerThread = 4;
static_assert(2 * kThreads * 16 == kStage4Rope && kThreads * 16 == kTok * kDr * 2 &&
                  32 * 16 == kTok * (kDc / kMxBlock),
              "4-bit stage must split into 16-byte loads");
static_assert(kStage4Bytes % 16 == 0, "4-bit stages start on 16-byte boundaries");

template <int kFmt>
struct StageFmt {
  static constexpr int bytes = kFmt == kFmtFp8 ? kStage8Bytes : (kFmt == kFmtMxfp4 ? kStage4Bytes : kStageBytes);
  static constexpr int dma = kFmt == kFmtFp8 ? kDma8PerThread : (kFmt == kFmtMxfp4 ? kDma4PerThread : kDmaPerThread);
  static constexpr int rope = kFmt == kFmtFp8 ? kStage8Rope : kStage4Rope;    // k_R rows (quantized formats)
  static constexpr int vbuf = kStages * bytes;                                // dequantized V tiles (4-bit)
  static constexpr int pbuf = vbuf + (kFmt == kFmtMxfp4 ? 2 * kStageBytes : 0);
  static constexpr int lds = pbuf + kPBytes;
};
static_assert(StageFmt<kFmtFp8>::lds <= 163840 && StageFmt<kFmtMxfp4>::lds <= 163840, "LDS budget");

__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) ^ ((t >> 2) & 7); }
// 8-bit stage: chunk c of code row t sits at c ^ swz8(t) (low 3 bits). Rows
// 0..7 of a run of eight differ in the low 3 bits and rows t, t+8 in bit 2, so
// both the 16-byte QK reads (eight consecutive rows) and the transposed
// 8-byte PV reads (rows 16ks + 8a + 4g + b, a < 2, b < 4) hit eight distinct
// 16-byte slots of a 128-byte line. k_R rows (128 bytes) use c ^ (t & 7).
__device__ __forceinline__ int swz8(int t) { return (t & 7) ^ ((t >> 1) & 4); }

// 8 E4M3 codes (byte j of d0:d1 = element j) -> 8 bf16 values times scale; the
// scale is a power of two, so every product is exact
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(unsigned d0, unsigned d1, float scale) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The lane id recomputed where it is used (two VALU ops). Written as
// volatile asm so the compiler cannot hoist lane-dependent addresses out of
// the piece loop, where they would be held, and spilled, across the tile loop.
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ float shfl_xor32(float v) { return __shfl_xor(v, 32, 64); }

// max(v[l], v[l ^ 32]) in every lane, on the VALU: v_permlane32_swap exchanges
// the upper half-wave of one register with the lower half of another (a
// copy of v), so each lane then holds both values of its pair. Unlike a
// cross-half shuffle it does not go through LDS, whose counter would also
// make the wait cover the LDS reads in flight. Written as asm with the wait
// states for its operands (the builtin loses its second result with this
// compiler).
__device__ __forceinline__ float pair_max32(float v) {
  float w = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1"
               : "+v"(v), "+v"(w));
  return v;
}

// S^T accumulation kept in VGPRs (the softmax reads it with VALU) while the
// 256 AGPRs hold O^T. Only this MFMA is written as asm: a chain whose srcC is
// exactly the previous destination needs no wait states.
__device__ __forceinline__ void mfma_qk_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_qk(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// The QK MFMAs are inline asm, so the compiler cannot see their hazards. A
// VALU read of a v_mfma_f32_32x32x16_bf16 result (8 passes) needs 12 wait
// states after the MFMA issues on gfx950: the count the compiler's own hazard
// model inserts after the builtin. MFMAs that accumulate onto the same
// registers (also a scaled f8f6f4 chain continued by bf16 MFMAs) need none.
// Tied to the value so no read of it can be scheduled above the wait.
__device__ __forceinline__ void mfma_result_fence(f32x16& d) {
  asm("s_nop 11" : "+v"(d));
}

// scheduling hint: one MFMA followed by up to N VALU/transcendental ops, four times
template <int N>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x402, N, 0);
  }
}

// Workgroup barrier for the tile pipeline: this wave's LDS writes are done
// (lgkmcnt 0) and the wave has already waited for its own direct-to-LDS loads
// of the tile with an explicit vmcnt. Unlike __syncthreads() it does not
// drain every outstanding global load (its release fence would wait for the
// whole prefetch window). The memory clobber keeps the compiler from moving
// memory operations across it.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One 16-byte-per-lane direct-to-LDS load: lane l's 16 bytes from
// sbase + voff land at LDS byte address lds_addr + 16*l. Written as asm so the
// compiler does not treat every later LDS read as possibly overlapping it
// (which would make it drain all outstanding loads); completion is tracked
// with explicit vmcnt waits before the tile is read. The LDS address is an
// operand bound to M0 ("{m0}"), so the compiler writes M0 itself and knows the
// register is taken; the s_nop is the one wait state an LDS-DMA instruction
// needs after an SALU write of M0.
// kStream: each cache row is read once per launch (one query row per
// sequence), so the loads are marked non-temporal (measured 2-4% faster:
// less cache fill traffic and power under the streaming load). With several
// query rows per sequence the same pages are read again by the other rows
// and the default policy keeps them in L2 and the last-level cache.
template <bool kStream>
__device__ __forceinline__ void dma16(const char* sbase, unsigned voff, unsigned lds_addr) {
  if constexpr (kStream)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr)
                 : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr)
                 : "memory");
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;
typedef short v2i16 __attribute__((ext_vector_type(2)));
typedef float v2f32 __attribute__((ext_vector_type(2)));

// 8-bit path: one lane's 16 query values of a 32-dim block (the block's other
// 16 are in lane l ^ 32) as two E4M3 terms with per-block power-of-two scales,
// q = hi * 2^kh + lo * 2^kl. hi keeps the top 4 significant bits of each bf16
// value (truncated, so the remainder has at most 4 significant bits and lo
// holds it exactly unless it falls below lo's subnormal range, i.e. for
// values under 2^-13 of the block's largest). Returns hi's 16 codes in h and
// lo's in l (byte j of the 16 = value j) and the two scale exponents.
__device__ __forceinline__ void split_block_fp8(const bf16x8& x0, const bf16x8& x1, u32x4& h, u32x4& l, int& kh,
                                                int& kl) {
  float v[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[j] = (float)x0[j];
    v[8 + j] = (float)x1[j];
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) amax = fmaxf(amax, __builtin_fabsf(v[j]));
  kh = fp8_scale_exponent(pair_max32(amax));
  // the scaled conversions divide by the scale on the way to E4M3 and multiply
  // on the way back; with a power of two both are exact, so the codes are those
  // of the value times 2^-kh (and the value back is hi * 2^kh), without the
  // separate ldexp of each element
  const float sh = __builtin_ldexpf(1.0f, kh);
  float r[16];
#pragma unroll
  for (int j = 0; j < 16; j += 4) {
    float t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = __uint_as_float(__float_as_uint(v[j + e]) & 0xFFF00000u);
    v2i16 c = {0, 0};
    c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, t[0], t[1], sh, false);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, t[2], t[3], sh, true);
    const unsigned cw = __builtin_bit_cast(unsigned, c);
    const v2f32 h0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw, sh, false);  // exact hi * 2^kh of the pairs
    const v2f32 h1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw, sh, true);
    r[j] = v[j] - h0[0];
    r[j + 1] = v[j + 1] - h0[1];
    r[j + 2] = v[j + 2] - h1[0];
    r[j + 3] = v[j + 3] - h1[1];
    h[j >> 2] = cw;
  }
  float rmax = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) rmax = fmaxf(rmax, __builtin_fabsf(r[j]));
  kl = fp8_scale_exponent(pair_max32(rmax));
  const float sl = __builtin_ldexpf(1.0f, kl);
#pragma unroll
  for (int j = 0; j < 16; j += 4) {
    v2i16 c = {0, 0};
    c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, r[j], r[j + 1], sl, false);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, r[j + 2], r[j + 3], sl, true);
    l[j >> 2] = __builtin_bit_cast(unsigned, c);
  }
}

// E4M3 x E4M3 scaled MFMA (32x32x64) accumulating into d, which stays in
// VGPRs (asm, as the bf16 QK chain): A's E8M0 scale is byte 0 of sa, B's is
// byte kSel of sb (op_sel / op_sel_hi of the second scale operand). A comes
// from LDS; the first MFMA of a tile carries the 2 wait states an MFMA needs
// after a VALU write of a source (the tile's token scale), later ones chain on
// the same d and need none.
template <int kSel, bool kFirst>
__device__ __forceinline__ void mfma_scaled_sel(f32x16& d, const i32x8& a, const i32x8& b, int sa, int sb) {
  if constexpr (kFirst) {
    if constexpr (kSel == 0)
      asm("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4" : "=&v"(d) : "v"(a), "v"(b), "v"(sa), "v"(sb));
    else if constexpr (kSel == 1)
      asm("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel:[0,1,0]"
          : "=&v"(d) : "v"(a), "v"(b), "v"(sa), "v"(sb));
    else if constexpr (kSel == 2)
      asm("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,1,0]"
          : "=&v"(d) : "v"(a), "v"(b), "v"(sa), "v"(sb));
    else
      asm("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
          : "=&v"(d) : "v"(a), "v"(b), "v"(sa), "v"(sb));
  } else {
    if constexpr (kSel == 0)
      asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4" : "+v"(d) : "v"(a), "v"(b), "v"(sa), "v"(sb));
    else if constexpr (kSel == 1)
      asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[0,1,0]"
          : "+v"(d) : "v"(a), "v"(b), "v"(sa), "v"(sb));
    else if constexpr (kSel == 2)
      asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,1,0]"
          : "+v"(d) : "v"(a), "v"(b), "v"(sa), "v"(sb));
    else
      asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
          : "+v"(d) : "v"(a), "v"(b), "v"(sa), "v"(sb));
  }
}
template <bool kFirst>
__device__ __forceinline__ void mfma_scaled(int sel, f32x16& d, const i32x8& a, const i32x8& b, int sa, int sb) {
  switch (sel) {
    case 0: mfma_scaled_sel<0, kFirst>(d, a, b, sa, sb); break;
    case 1: mfma_scaled_sel<1, kFirst>(d, a, b, sa, sb); break;
    case 2: mfma_scaled_sel<2, kFirst>(d, a, b, sa, sb); break;
    default: mfma_scaled_sel<3, kFirst>(d, a, b, sa, sb); break;
  }
}

// E2M1 x E4M3 scaled MFMA (32x32x64, cbsz 4: A is 4-bit) accumulating into d
// in VGPRs. A = 32 tokens x 64 latent dims of 4-bit codes: lane half g holds
// all 32 values of the MFMA's K-block g (byte j = K values 2j, 2j+1, low
// nibble first), with that block's E8M0 scale; B as in the 8-bit scan. Both
// scales are byte kSel of their registers. kInit: d = A.B (srcC 0); kNop: two
// wait states first, for a source written by the VALU just before.
template <int kSel, bool kInit, bool kNop>
__device__ __forceinline__ void mfma_scaled4_sel(f32x16& d, const u32x4& a, const i32x8& b, int sa, int sb) {
#define MLA_SEL4(OPS) \
  if constexpr (kInit) \
    asm("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4" OPS " cbsz:4" \
        : "=&v"(d) : "v"(a), "v"(b), "v"(sa), "v"(sb)); \
  else if constexpr (kNop) \
    asm("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4" OPS " cbsz:4" \
        : "+v"(d) : "v"(a), "v"(b), "v"(sa), "v"(sb)); \
  else \
    asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4" OPS " cbsz:4" \
        : "+v"(d) : "v"(a), "v"(b), "v"(sa), "v"(sb));
  if constexpr (kSel == 0) {
    MLA_SEL4("")
  } else if constexpr (kSel == 1) {
    MLA_SEL4(" op_sel:[1,1,0]")
  } else if constexpr (kSel == 2) {
    MLA_SEL4(" op_sel_hi:[1,1,0]")
  } else {
    MLA_SEL4(" op_sel:[1,1,0] op_sel_hi:[1,1,0]")
  }
#undef MLA_SEL4
}

__device__ __forceinline__ bf16x8 cat8(const i16x4& v0, const i16x4& v1) {
  const bf16x4 b0 = __builtin_bit_cast(bf16x4, v0);
  const bf16x4 b1 = __builtin_bit_cast(bf16x4, v1);
  return bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
}

// Split-plan arithmetic counts pages in 32 bits: the host rejects launches
// with B * s_q * max_pages >= 2^31, which bounds every sum below.
// Pages of keys 1..x summed over rows: sum_{v=1..x} ceil(v / 64) (0 for x <= 0).
__device__ __forceinline__ int pages_prefix(int x) {
  if (x <= 0) return 0;
  const int q = x >> 6, r = x & (kPage - 1);
  return kPage * q * (q + 1) / 2 + r * (q + 1);
}
// Pages of the first i query rows of a sequence holding L tokens: row i' sees
// L - s_q + i' + 1 keys.
__device__ __forceinline__ int rows_pages(int L, int s_q, int i) {
  return pages_prefix(L - s_q + i) - pages_prefix(L - s_q);
}
// Inclusive prefix sum (or running max) over the 64 lanes on DPP: shifts by 1,
// 2, 4 and 8 lanes inside each 16-lane row, then lane 15's value into rows 1
// and 3 and lane 31's into rows 2 and 3 (the two row broadcasts of the GFX9
// DPP set). Six dependent VALU steps and no LDS round trip, where a __shfl
// ladder costs one ds_bpermute round trip per step; the plan runs three of
// these before a piece can start. Lanes shifted in read 0, so v must be >= 0
// (page counts).
template <bool kMax>
__device__ __forceinline__ int wave_scan_dpp(int v) {
  auto step = [&](int u) { v = kMax ? max(v, u) : v + u; };
  step(__builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true));   // row_shr:1
  step(__builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true));   // row_shr:2
  step(__builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true));   // row_shr:4
  step(__builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true));   // row_shr:8
  step(__builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  step(__builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return v;
}
__device__ __forceinline__ int wave_sum32(int v) { return __builtin_amdgcn_readlane(wave_scan_dpp<false>(v), 63); }
__device__ __forceinline__ int wave_max32(int v) { return __builtin_amdgcn_readlane(wave_scan_dpp<true>(v), 63); }
__device__ __forceinline__ int wave_incl_scan32(int v) { return wave_scan_dpp<false>(v); }

}  // namespace

// kFmt: the cache is bf16 rows (kFmtBf16), the 8-bit layout of fp8_cache.hpp
// (kFmtFp8) or the 4-bit layout of mxfp4_cache.hpp (kFmtMxfp4).
// 8-bit:
// QK over the latent runs on the E4M3 block-scaled MFMA straight from the
// codes (the token's scale as A's block scale); the query is held as two E4M3
// terms, hi (each bf16 value truncated to 4 significant bits) and lo (the
// remainder), with per-32-dim block scales, which reproduce it exactly except
// for values under 2^-13 of their block's largest. PV converts a V^T fragment
// (8 tokens of one column, read transposed) to bf16 at scale 1 and folds the
// tokens' scales into P (P' = P * 2^k_t is exact).
// The body of one scan workgroup (blockIdx.x is its range); lds points at
// decode_lds_bytes<kFmt>() bytes of LDS aligned to 1024. It runs as its own
// kernel (decode.hip) and as a phase of the fused step (step.hip).
template <bool kStream, int kFmt>
__device__ __forceinline__ void decode_paged_body(
    char* __restrict__ lds, const __bf16* __restrict__ q_abs, const __bf16* __restrict__ q_r,
    const char* __restrict__ kv, const int32_t* __restrict__ block_table, const int32_t* __restrict__ seqlens,
    float* __restrict__ o_part, float* __restrict__ lse_part, DecodeParams a) {
  constexpr bool kFp8 = kFmt == kFmtFp8;
  constexpr bool kFp4 = kFmt == kFmtMxfp4;
  constexpr bool kScaled = kFp8 || kFp4;  // QK over the latent on the block-scaled MFMA
  using F = StageFmt<kFmt>;
  char* const pbuf = lds + F::pbuf;
  char* const vbuf = lds + F::vbuf;  // 4-bit cache: two dequantized V tiles

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lo = lane & 31;
  const int g = lane >> 5;

  // ---- split plan: the pages of all rows (b, i), concatenated in order, are
  // cut into kScanGroups equal ranges of W pages; workgroup k scans range k
  // and writes one partial for every row piece in it, into slot
  // k - floor(P_r / W) of row r (P_r = the row's first page in the
  // concatenation). W is at least ceil((n_max - 1) / (num_splits - 1)), so a
  // row never needs more than num_splits slots; with num_splits = 1 rows are
  // not cut and each row goes whole to the range holding its middle page
  // (first page + floor(n / 2)): rows of nearly equal length then spread
  // evenly, and the workgroups of an XCD start their rows at the same page,
  // so a chunk's query rows, which all rescan one prefix, share it in L2.
  const int S = a.num_splits;
  // the first 64 sequences stay in registers (lane = sequence); larger
  // batches are read in further blocks of 64
  const int L0 = lane < a.B ? clamp_len(seqlens[lane], a.max_pages) : 0;
  const int T0 = lane < a.B ? rows_pages(L0, a.s_q, a.s_q) : 0;
  int p_tot = wave_sum32(T0);
  int n_max = wave_max32((L0 + kPage - 1) / kPage);
  bool any_empty_row = __any(lane < a.B && L0 < a.s_q);
  for (int b0 = 64; b0 < a.B; b0 += 64) {
    const int bb = b0 + lane;
    const int L = bb < a.B ? clamp_len(seqlens[bb], a.max_pages) : 0;
    p_tot += wave_sum32(bb < a.B ? rows_pages(L, a.s_q, a.s_q) : 0);
    n_max = max(n_max, wave_max32((L + kPage - 1) / kPage));
    any_empty_row |= __any(bb < a.B && L < a.s_q);
  }
  int W = (p_tot + kScanGroups - 1) / kScanGroups;
  if (S > 1) W = max(W, (n_max - 1 + S - 2) / (S - 1));
  if (W < 1) W = 1;
  // the ceil(p_tot / W) non-empty ranges are dealt contiguously over all 8
  // XCDs (workgroups go to the XCDs round-robin), so a sequence's pieces
  // share an L2 for its queries and every XCD's bandwidth is used
  const int n_ranges = (p_tot + W - 1) / W;
  const int per_xcd = (n_ranges + 7) / 8;
  const bool has_range = (int)(blockIdx.x >> 3) < per_xcd;
  const int k = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int r_lo = has_range ? k * W : p_tot;  // k * W < p_tot + W <= 2^31
  const int r_hi = min(r_lo + W, p_tot);

  // rows that see no key at all: every slot's LSE is -inf; row r is written
  // by workgroup (blockIdx) r mod kScanGroups
  if (any_empty_row) {
    for (int bb = 0; bb < a.B; ++bb) {
      const int L = clamp_len(seqlens[bb], a.max_pages);
      for (int ii = 0; ii < a.s_q - L; ++ii) {
        const int64_t r = (int64_t)bb * a.s_q + ii;
        if (r % kScanGroups != (int)blockIdx.x) continue;
        for (int q = tid; q < kH * S; q += kThreads) lse_part[r * kH * S + q] = -INFINITY;
      }
    }
  }
  if (r_lo >= r_hi) return;

  // first row touching the range: the sequence whose pages end past r_lo, then
  // (binary search) its last query row starting at or before r_lo
  int cb = 0, cL = 0;
  int cp = 0;  // first page of sequence cb
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int bb = b0 + lane;
    const int L = b0 == 0 ? L0 : (bb < a.B ? clamp_len(seqlens[bb], a.max_pages) : 0);
    const int t = b0 == 0 ? T0 : (bb < a.B ? rows_pages(L, a.s_q, a.s_q) : 0);
    const int incl = wave_incl_scan32(t);
    const uint64_t hit = __ballot(cp + incl > r_lo);
    if (hit) {
      const int f = __builtin_ctzll(hit);
      cb = b0 + f;
      cL = __builtin_amdgcn_readlane(L, f);
      cp += __builtin_amdgcn_readlane(incl - t, f);
      break;
    }
    cp += __builtin_amdgcn_readlane(incl, 63);
  }
  int ci = 0;
  {
    int lo_i = 0, hi_i = a.s_q - 1;  // largest i with cp + rows_pages(cL, s_q, i) <= r_lo
    while (lo_i < hi_i) {
      const int mid = (lo_i + hi_i + 1) >> 1;
      if (cp + rows_pages(cL, a.s_q, mid) <= r_lo) lo_i = mid; else hi_i = mid - 1;
    }
    ci = lo_i;
    cp += rows_pages(cL, a.s_q, ci);
  }

  // per-piece state, set by the piece loop at the end of the kernel
  int b = 0, i = 0, split = 0, tile0 = 0, t_end = 0, n_tiles = 0;
  int64_t qbase = 0;  // row of head 0 of the piece's query
  const int h_own = wave * 32 + lo;                       // head this lane owns in QK/softmax

  // QK A operand: row lo, chunk 2kk+g; kk = 4a + r -> offset qk_off[r] + 128a
  int qk_off[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) qk_off[r] = lo * kRowBytes + (((2 * r + g) ^ swz(lo)) << 4);
  // 8-bit: the K operand of scaled MFMA m (latent dims 64m .. 64m + 63) is code
  // chunks 4m + g (dims 64m + 16g .. +15, first K-block) and 4m + 2 + g (dims
  // 64m + 32 + 16g .. +15, second K-block) of row lo, at
  // qk8_off[2(m & 1) + p] + 128 (m >> 1) for p = 0, 1; k_R chunk 2r' + g at
  // rope8_off + ((32 r') ^ rope8_x)
  int qk8_off[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) qk8_off[r] = lo * kDc + (((4 * (r >> 1) + 2 * (r & 1) + g) ^ swz8(lo)) << 4);
  // 4-bit: the A operand of scaled MFMA m is code chunk 2m + g of row lo (all
  // of MX block 2m + g), at chunk slot (2m + g) ^ (lo & 7) =
  // 2((m & 3) ^ ((lo >> 1) & 3)) + (g ^ (lo & 1)) + 8 (m >> 2): qk4_off[m & 3] + 128 (m >> 2)
  int qk4_off[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    qk4_off[r] = lo * kFp4RowBytes + (((2 * (r ^ ((lo >> 1) & 3))) + (g ^ (lo & 1))) << 4);
  const int rope8_off = F::rope + lo * (kDr * 2);
  const int rope8_x = (g ^ (lo & 7)) << 4;
  // PV A operand (V^T) for this wave's columns 128w + 32c' through transposed
  // reads; group G = lane>>4, ii = lane&15 fetches row 4(G>>1) + (ii>>2)
  // (+8 half, +16 k-step), columns 16(G&1) + 4(ii&3)..+3 of the 32-column tile.
  int pv_off[2][2][2];  // [c'&1][half][k-step]; add (c'>>1)*128
  {
    const int G = lane >> 4, ii = lane & 15;
    const int t_lane = 4 * (G >> 1) + (ii >> 2);
    const int jl = 2 * (G & 1) + ((ii & 3) >> 1);
#pragma unroll
    for (int cp = 0; cp < 2; ++cp)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int t = t_lane + 8 * hf + 16 * ks;
          const int j = 4 * cp + jl;
          pv_off[cp][hf][ks] = t * kRowBytes + ((j ^ swz(t)) << 4) + (ii & 1) * 8 + wave * 256;
        }
  }
  // 8-bit PV A operand through ds_read_b64_tr_b8: in each 16-lane group G,
  // lane 8h + j receives byte j of the 8 bytes that lanes 2k + h of the group
  // address, as its element k. Lane (G, k, h) therefore addresses row
  // 4(G>>1) + 8(k>>2) + (k&3) (+16 per k-step), columns 16(G&1) + 8h .. +7 of
  // the 32-column tile: lane l then holds column l&31 for the tokens of
  // k-slot j = 8(l>>5)... order that P^T uses (16ks + 8(j>>2) + 4(l>>5) + (j&3)).
  int pv8_off[4];  // [c']; add 8192 (16 rows) for k-step 1
  {
    const int G = lane >> 4, kq = (lane & 15) >> 1, h = lane & 1;
    const int t = 8 * (kq >> 2) + 4 * (G >> 1) + (kq & 3);
#pragma unroll
    for (int cp = 0; cp < 4; ++cp)
      pv8_off[cp] = t * kDc + wave * 128 + (((2 * cp + (G & 1)) ^ swz8(t)) << 4) + 8 * h;
  }
  // DMA: thread tid fills chunk slot q = k*256 + tid of a stage; the matching
  // source chunk of the 32-row half page is (row q/72, chunk (q%72) ^ swz(row))
  unsigned dma_off[F::dma];
  if constexpr (kFp4) {
    // code slot q = k*256 + tid (k < 2): row q/16, source chunk (q%16) ^ (row&7);
    // k_R slot tid as in the 8-bit stage; scale slot 8*wave + lane (lanes 0-7)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const unsigned q = k * kThreads + tid;
      const unsigned t = q >> 4;
      dma_off[k] = t * kFp4RowBytes + (((q & 15) ^ (t & 7)) << 4);
    }
    dma_off[2] = (tid >> 3) * (kDr * 2) + (((tid & 7) ^ ((tid >> 3) & 7)) << 4);
    dma_off[3] = (8 * wave + (tid & 7)) * 16;
  } else if constexpr (kFp8) {
    // code slot q = k*256 + tid (k < 4): row q/32, source chunk (q%32) ^ swz8(row);
    // k_R slot tid: row tid/8, source chunk (tid%8) ^ (row&7); scale slot
    // 2*wave + lane (lanes 0-1)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const unsigned q = k * kThreads + tid;
      const unsigned t = q >> 5;
      dma_off[k] = t * kDc + (((q & 31) ^ swz8(t)) << 4);
    }
    dma_off[4] = (tid >> 3) * (kDr * 2) + (((tid & 7) ^ ((tid >> 3) & 7)) << 4);
    dma_off[5] = (2 * wave + (tid & 1)) * 16;
  } else {
#pragma unroll
    for (int k = 0; k < kDmaPerThread; ++k) {
      const unsigned q = k * kThreads + tid;
      const unsigned t = q / 72u;
      const unsigned p = q - t * 72u;
      dma_off[k] = t * kRowBytes + ((p ^ swz(t)) << 4);
    }
  }
  // DMA of one 32-token tile (half a page) into an LDS stage, 9 loads per
  // thread; issue_part(k) issues load k so the loads can be spread between
  // the MFMAs of the QK phase.
  struct DmaTarget {
    const char* src;
    unsigned dst;
  };
  // 8-bit: src is the page's first byte, dst the stage's wave slice
  auto page_target = [&](int64_t page, int tile, int stage) -> DmaTarget {
    if constexpr (kFp4)
      return DmaTarget{kv + page * kFp4PageBytes,
                       (unsigned)(uintptr_t)(lds_void_t*)(lds + stage * F::bytes + wave * 1024)};
    else if constexpr (kFp8)
      return DmaTarget{kv + page * kFp8PageBytes,
                       (unsigned)(uintptr_t)(lds_void_t*)(lds + stage * F::bytes + wave * 1024)};
    else
      return DmaTarget{kv + page * kPageBytes + (tile & 1) * kStageBytes,
                       (unsigned)(uintptr_t)(lds_void_t*)(lds + stage * kStageBytes + wave * 1024)};
  };
  auto dma_target = [&](int tile, int stage) -> DmaTarget {
    return page_target(physical_page(block_table, a.max_pages, b, tile >> 1, a.num_pages), tile, stage);
  };
  // load k of a tile (k is a compile-time constant at every call); the 8-bit
  // tile is half `tile & 1` of its page in each of the page's three arrays
  auto dma_piece = [&](const DmaTarget& t, int k, int tile) {
    if constexpr (kFp4) {
      const int half = tile & 1;
      if (k < 2) {
        dma16<kStream>(t.src + half * (kTok * kFp4RowBytes), dma_off[k], t.dst + k * (kThreads * 16));
      } else if (k == 2) {
        dma16<kStream>(t.src + kFp4RopeOffset + half * (kTok * kDr * 2), dma_off[2], t.dst + kStage4Rope);
      } else if ((tid & 63) < 8) {
        dma16<kStream>(t.src + kFp4ScaleOffset + half * (kTok * (kDc / kMxBlock)), dma_off[3],
                       t.dst - wave * 1024 + kStage4Scale + wave * 128);
      }
    } else if constexpr (kFp8) {
      const int half = tile & 1;
      if (k < 4) {
        dma16<kStream>(t.src + half * (kTok * kDc), dma_off[k], t.dst + k * (kThreads * 16));
      } else if (k == 4) {
        dma16<kStream>(t.src + kFp8RopeOffset + half * (kTok * kDr * 2), dma_off[4], t.dst + kStage8Rope);
      } else if ((tid & 63) < 2) {
        dma16<kStream>(t.src + kFp8ScaleOffset + half * (kTok * 4), dma_off[5],
                       t.dst - wave * 1024 + kStage8Scale + wave * 32);
      }
    } else {
      dma16<kStream>(t.src, dma_off[k], t.dst + k * (kThreads * 16));
    }
  };
  auto issue = [&](int tile, int stage) {
    const DmaTarget t = dma_target(tile, stage);
#pragma unroll
    for (int k = 0; k < F::dma; ++k) dma_piece(t, k, tile);
  };

  bf16x8 qf[36];  // queries of the current piece (8-bit path: only the k_R part, qf[32..35])
  // 8-bit: the B operands of scaled MFMA m, hi codes in qhl[2m] and lo codes in
  // qhl[2m+1], and byte m & 3 of qsh / qsl [m >> 2] their E8M0 scales
  i32x8 qhl[16];
  int qsh[2] = {0, 0}, qsl[2] = {0, 0};

  const float c_log2 = a.scale_log2;
  f32x16 O[4][4];            // O^T tiles [column tile c'][head tile ht]
  float m_ref = -INFINITY;   // reference max of head h_own (log2 units)
  float m_seen = -INFINITY;  // true running max of head h_own
  float l_run = 0.f;         // this lane's share of sum exp2(x - m_ref)

  // ---- PV pieces: V^T fragment (k-step ks, column tile c') and P^T fragment
  // (k-step ks, head tile ht) of tile ip, and the 4 MFMAs of one (ks, c')
  // a V^T fragment as read from LDS: bf16 values, or for the 8-bit cache the
  // 8 codes of one transposed read, converted (scale 1) right before its MFMAs
  using VFrag = std::conditional_t<kFp8, i32x2, bf16x8>;
  auto vop = [&](const VFrag& v) -> bf16x8 {
    if constexpr (kFp8)
      return fp8x8_to_bf16((unsigned)v[0], (unsigned)v[1], 1.0f);
    else
      return v;
  };
  auto vfrag = [&](int ip, int ks, int cp) -> VFrag {
    if constexpr (kFp8) {
      const char* tv = lds + (ip & (kStages - 1)) * F::bytes + pv8_off[cp] + ks * (16 * kDc);
      return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)tv);
    } else {
      const char* tv = (kFp4 ? vbuf + (ip & 1) * kStageBytes : lds + (ip & (kStages - 1)) * kStageBytes) +
                       (cp >> 1) * 128;
      return cat8(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(tv + pv_off[cp & 1][0][ks])),
                  __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(tv + pv_off[cp & 1][1][ks])));
    }
  };
  auto pfrag = [&](int ip, int ks, int ht) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(pbuf + (ip & 1) * 8 * 1024 + (ht * 2 + ks) * 1024 + lane * 16);
  };
  auto mm4 = [&](int cp, const VFrag& vf, const bf16x8* pf) {
    const bf16x8 va = vop(vf);
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
      O[cp][ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[ht], O[cp][ht], 0, 0, 0);
  };
  // PV operands, carried across iterations: PV(i) leaves its last four
  // MFMAs (k-step 1, column tile 3) to run right after the next tile
  // barrier, where they cover the latency of the first K reads of QK(i+2);
  // zero operands (a no-op MFMA) when there is no earlier tile
  bf16x8 pf[4];
  VFrag va[3];
  // Block-table entry of the page that QK(it) streams in (tile it + 2), loaded
  // during the P publish of tile it - 1, so the scalar load has returned by
  // the tile barrier; looked up right after the barrier, its latency and the
  // clamp stood between the barrier and the tile's first MFMA (A/B,
  // bit-identical: long 267.7 -> 266.1 us, 8-bit 262.3 -> 258.5 us). The
  // clamp is physical_page's, on 32-bit scalar min/max (ids are 32-bit).
  int pref_id = 0;
  const int last_page = (int)(a.num_pages - 1 < (int64_t)0x7fffffff ? a.num_pages - 1 : (int64_t)0x7fffffff);
  auto load_id = [&](int tile) { return block_table[(int64_t)b * a.max_pages + (tile >> 1)]; };
  auto pref_target = [&](int tile, int stage) {
    return page_target((int64_t)min(max(pref_id, 0), last_page), tile, stage);
  };

  // ---- phase A: S^T[token, head] = K(it) . Q^T over 576 dims, pinned in
  // program order: the K fragment for MFMA kk+3 is read right after MFMA kk,
  // so three LDS reads are always in flight.
  // The next tile's DMA (if any) is issued inside the QK phase, one load
  // after every fourth MFMA, so the issue cost hides under matrix-core work.
  // dma_tag is std::true_type / std::false_type: whether to issue DMA(it+2).
  auto qk = [&](int it, auto dma_tag, auto pv_tag) -> f32x16 {
    constexpr bool dma = decltype(dma_tag)::value;
    constexpr bool pv = decltype(pv_tag)::value;  // prefetch PV(it-1) operands
    if constexpr (kFp4) {
      // 4-bit: the latent part on v_mfma_scale_f32_32x32x64_f8f6f4 with A =
      // the tile's E2M1 codes and their per-token, per-block E8M0 scales
      // (lane half g supplies K-block g: all of MX block 2m + g), B = the
      // query's E4M3 hi and lo terms as in the 8-bit scan; then the four bf16
      // MFMAs of k_R. Inside every MFMA pair each thread dequantizes one
      // 16-byte chunk of its eighth of V(it) (token tid & 31, dims
      // 64 (tid >> 5) .. +63) into the bf16 tile vbuf[it & 1]; in the tail
      // tile the rows past the visible length are then overwritten with zeros.
      const char* tb = lds + (it & (kStages - 1)) * F::bytes;
      DmaTarget t{nullptr, 0u};
      if constexpr (dma) t = pref_target(tile0 + it + 2, (it + 2) & (kStages - 1));
      // A scales: byte m & 3 of sa[m >> 2] = scale of MX block 2m + g of token lo
      int sa[2];
      {
        const u32x4 w = *reinterpret_cast<const u32x4*>(tb + kStage4Scale + lo * 16);
        const unsigned sel = 0x06040200u + 0x01010101u * (unsigned)g;
        sa[0] = (int)__builtin_amdgcn_perm(w[1], w[0], sel);
        sa[1] = (int)__builtin_amdgcn_perm(w[3], w[2], sel);
      }
      auto kread = [&](int m) -> u32x4 {
        return *reinterpret_cast<const u32x4*>(tb + qk4_off[m & 3] + 128 * (m >> 2));
      };
      // V dequantization of this thread's token dt and dims 64 ds .. 64 ds + 63
      const int dl = lane_here();
      const int dt = dl & 31;
      const int ds = 2 * wave + (dl >> 5);
      const u32x4 dc0 = *reinterpret_cast<const u32x4*>(tb + dt * kFp4RowBytes + (((2 * ds) ^ (dt & 7)) << 4));
      const u32x4 dc1 = *reinterpret_cast<const u32x4*>(tb + dt * kFp4RowBytes + (((2 * ds + 1) ^ (dt & 7)) << 4));
      const unsigned de = *reinterpret_cast<const unsigned short*>(tb + kStage4Scale + dt * 16 + 2 * ds);
      // chunk 8 ds + j of the row sits at slot (8 ds + j) ^ swz(dt) = 8 ds + (j ^ swz(dt)) (swz < 8):
      // from an offset whose bits 0-6 are zero but for the swizzle in bits 4-6, each chunk's
      // address is one XOR (21 fewer VALU ops per wave and tile than recomputing the slot;
      // long workload 245.8 -> 239.7 us, bit-identical)
      static_assert(F::vbuf % 128 == 0 && kStageBytes % 128 == 0 && kRowBytes % 128 == 0, "128-byte aligned rows");
      const int vrel = F::vbuf + (it & 1) * kStageBytes + dt * kRowBytes + 128 * ds + (swz(dt) << 4);
      auto dequant = [&](int j) {  // output chunk 8 ds + j (dims 64 ds + 8j .. +7)
        const unsigned w = (j < 4 ? dc0 : dc1)[j & 3];
        const float sc = __uint_as_float(((j < 4 ? de : de >> 8) & 255u) << 23);
        const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
        const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
        const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
        const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
        *reinterpret_cast<bf16x8*>(lds + (vrel ^ (j << 4))) =
            bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
      };
      u32x4 ka[2];
      ka[0] = kread(0);
      __builtin_amdgcn_sched_barrier(0);
      mm4(3, va[1], pf);  // deferred tail of the previous PV
      __builtin_amdgcn_sched_barrier(0);
      f32x16 S;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m + 1 < 8) ka[(m + 1) & 1] = kread(m + 1);  // one MFMA pair ahead
        if (m == 0)
          mfma_scaled4_sel<0, true, true>(S, ka[0], qhl[0], sa[0], qsh[0]);
        else if (m == 4)
          mfma_scaled4_sel<0, false, true>(S, ka[0], qhl[8], sa[1], qsh[1]);
        else if ((m & 3) == 1)
          mfma_scaled4_sel<1, false, false>(S, ka[m & 1], qhl[2 * m], sa[m >> 2], qsh[m >> 2]);
        else if ((m & 3) == 2)
          mfma_scaled4_sel<2, false, false>(S, ka[m & 1], qhl[2 * m], sa[m >> 2], qsh[m >> 2]);
        else
          mfma_scaled4_sel<3, false, false>(S, ka[m & 1], qhl[2 * m], sa[m >> 2], qsh[m >> 2]);
        // The second MFMA of the pair accumulates onto the first, so the wave
        // cannot issue it (or anything after it) until the first is done: VALU
        // work placed here issues while the first MFMA runs, work placed after
        // the second while the second runs.
        __builtin_amdgcn_sched_barrier(0);
        dequant(m);
        __builtin_amdgcn_sched_barrier(0);
        if ((m & 3) == 0)
          mfma_scaled4_sel<0, false, false>(S, ka[m & 1], qhl[2 * m + 1], sa[m >> 2], qsl[m >> 2]);
        else if ((m & 3) == 1)
          mfma_scaled4_sel<1, false, false>(S, ka[m & 1], qhl[2 * m + 1], sa[m >> 2], qsl[m >> 2]);
        else if ((m & 3) == 2)
          mfma_scaled4_sel<2, false, false>(S, ka[m & 1], qhl[2 * m + 1], sa[m >> 2], qsl[m >> 2]);
        else
          mfma_scaled4_sel<3, false, false>(S, ka[m & 1], qhl[2 * m + 1], sa[m >> 2], qsl[m >> 2]);
        if constexpr (dma) {
          if (m < F::dma) dma_piece(t, m, tile0 + it + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8 rf[2];
      rf[0] = *reinterpret_cast<const bf16x8*>(tb + rope8_off + (0 ^ rope8_x));
      // the tail tile: this thread's rows past the visible length become zeros
      // (written after its own chunks, and LDS writes of a wave land in order)
      if ((tile0 + it + 1) * kTok > t_end && (tile0 + it) * kTok + dt >= t_end) {
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<bf16x8*>(lds + (vrel ^ (j << 4))) = bf16x8{};
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r + 1 < 4) rf[(r + 1) & 1] = *reinterpret_cast<const bf16x8*>(tb + rope8_off + ((32 * (r + 1)) ^ rope8_x));
        mfma_qk(S, rf[r & 1], qf[32 + r]);
        if constexpr (pv) {
          if (r == 1) { pf[0] = pfrag(it - 1, 0, 0); pf[1] = pfrag(it - 1, 0, 1); }
          if (r == 2) { pf[2] = pfrag(it - 1, 0, 2); pf[3] = pfrag(it - 1, 0, 3); }
          if (r == 3) { va[0] = vfrag(it - 1, 0, 0); va[1] = vfrag(it - 1, 0, 1); }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_result_fence(S);
      __builtin_amdgcn_sched_barrier(0);
      return S;
    } else if constexpr (kFp8) {
      // 8-bit: the latent part runs on v_mfma_scale_f32_32x32x64_f8f6f4 straight
      // from the codes: A = 64 dims of the tile's K codes with the token's own
      // E8M0 scale, B = the same dims of the query's hi and lo code terms with
      // their per-32-dim block scales (two MFMAs per 64 dims, the time of the
      // four bf16 MFMAs they replace, and no conversion of K); then the four
      // bf16 MFMAs of k_R. K operands are read one MFMA pair ahead.
      const char* tb = lds + (it & (kStages - 1)) * F::bytes;
      DmaTarget t{nullptr, 0u};
      if constexpr (dma) t = pref_target(tile0 + it + 2, (it + 2) & (kStages - 1));
      // the token's scale 2^k as its E8M0 byte k + 127 (the exponent field)
      const int kscale = (int)(__float_as_uint(*reinterpret_cast<const float*>(tb + kStage8Scale + lo * 4)) >> 23);
      auto kread = [&](int m) -> i32x8 {
        const u32x4 c0 = *reinterpret_cast<const u32x4*>(tb + qk8_off[2 * (m & 1)] + 128 * (m >> 1));
        const u32x4 c1 = *reinterpret_cast<const u32x4*>(tb + qk8_off[2 * (m & 1) + 1] + 128 * (m >> 1));
        return i32x8{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
      };
      i32x8 ka[2];
      ka[0] = kread(0);
      __builtin_amdgcn_sched_barrier(0);
      mm4(3, va[1], pf);  // deferred tail of the previous PV
      __builtin_amdgcn_sched_barrier(0);
      f32x16 S;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m + 1 < 8) ka[(m + 1) & 1] = kread(m + 1);  // one MFMA pair ahead
        if (m == 0)
          mfma_scaled<true>(m & 3, S, ka[m & 1], qhl[2 * m], kscale, qsh[m >> 2]);
        else
          mfma_scaled<false>(m & 3, S, ka[m & 1], qhl[2 * m], kscale, qsh[m >> 2]);
        // the lo MFMA accumulates onto the hi one: the DMA issues while hi runs
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (dma) {
          if (m < F::dma) dma_piece(t, m, tile0 + it + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_scaled<false>(m & 3, S, ka[m & 1], qhl[2 * m + 1], kscale, qsl[m >> 2]);
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8 rf[2];
      rf[0] = *reinterpret_cast<const bf16x8*>(tb + rope8_off + (0 ^ rope8_x));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r + 1 < 4) rf[(r + 1) & 1] = *reinterpret_cast<const bf16x8*>(tb + rope8_off + ((32 * (r + 1)) ^ rope8_x));
        mfma_qk(S, rf[r & 1], qf[32 + r]);
        if constexpr (pv) {
          if (r == 1) { pf[0] = pfrag(it - 1, 0, 0); pf[1] = pfrag(it - 1, 0, 1); }
          if (r == 2) { pf[2] = pfrag(it - 1, 0, 2); pf[3] = pfrag(it - 1, 0, 3); }
          if (r == 3) { va[0] = vfrag(it - 1, 0, 0); va[1] = vfrag(it - 1, 0, 1); }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_result_fence(S);
      __builtin_amdgcn_sched_barrier(0);
      return S;
    }
    const char* tb = lds + (it & (kStages - 1)) * kStageBytes;
    DmaTarget t{nullptr, 0u};
    if constexpr (dma) t = pref_target(tile0 + it + 2, (it + 2) & (kStages - 1));
    f32x16 S;
    bf16x8 kf[4];
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) kf[kk] = *reinterpret_cast<const bf16x8*>(tb + qk_off[kk]);
    __builtin_amdgcn_sched_barrier(0);
    mm4(3, va[1], pf);  // deferred tail of the previous PV
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 36; ++kk) {
      if (kk == 0)
        mfma_qk_first(S, kf[0], qf[0]);
      else
        mfma_qk(S, kf[kk & 3], qf[kk]);
      if (kk + 3 < 36) {
        kf[(kk + 3) & 3] = *reinterpret_cast<const bf16x8*>(tb + qk_off[(kk + 3) & 3] + ((kk + 3) >> 2) * 128);
      } else if constexpr (pv) {
        // the K reads are done: fetch the first PV(it-1) operands instead
        if (kk == 33) { pf[0] = pfrag(it - 1, 0, 0); pf[1] = pfrag(it - 1, 0, 1); }
        if (kk == 34) { pf[2] = pfrag(it - 1, 0, 2); pf[3] = pfrag(it - 1, 0, 3); }
        if (kk == 35) { va[0] = vfrag(it - 1, 0, 0); va[1] = vfrag(it - 1, 0, 1); }
      }
      if constexpr (dma) {
        if (kk % kDmaGap == kDmaGap - 1 && kk / kDmaGap < kDmaPerThread) dma_piece(t, kk / kDmaGap, tile0 + it + 2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_result_fence(S);
    __builtin_amdgcn_sched_barrier(0);
    return S;
  };

  // ---- softmax numerators in chunks (lane owns head h_own and tokens
  // 8(r>>2) + 4g + (r&3) of the tile); chunks are interleaved with PV below
  float xs[16];
  float mx = 0.f;
  bf16x8 pb[2];
  // xs = raw scores; the tail tile masks tokens past the visible length.
  // kMay (a compile-time flag) is false where the tile is known to be full
  // (every tile at least two before the piece's last), so those tiles carry
  // no masking code at all: as a uniform runtime branch the compiler turns it
  // into 33 selects per tile.
  auto sm_scale = [&](const f32x16& S, int it, auto may_tag) {
    constexpr bool kMay = decltype(may_tag)::value;
    const int valid = t_end - (tile0 + it) * kTok;  // uniform; >= 32 for full tiles
#pragma unroll
    for (int r = 0; r < 16; ++r) xs[r] = S[r];
    if (kMay && valid < kTok) {
      const int vlim = valid - 4 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r) xs[r] = (8 * (r >> 2) + (r & 3)) < vlim ? xs[r] : -INFINITY;
    }
  };
  auto sm_localmax = [&]() {
    mx = fmaxf(fmaxf(xs[0], xs[1]), xs[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, xs[r]), xs[r + 1]);
    mx = fmaxf(mx, xs[15]);
    mx = pair_max32(mx);
  };
  // reference and running max in log2 units (softmax_scale > 0, so the max of
  // the scaled scores is the scaled max)
  auto sm_ref = [&](bool& over) {
    mx = mx * c_log2;
    m_seen = fmaxf(m_seen, mx);
    m_ref = m_ref == -INFINITY ? mx : m_ref;  // first tile of the first pass
    over |= mx > m_ref + kRefSlack;
  };
  // exp2(x*c - m_ref) in one fma: the exact product is used, so the weight of
  // the maximum itself is 2^e with |e| <= 2^-24 |m_ref| rather than exactly 1
  // 8-bit: P' = P * (scale of the token), exact since the scale is a power of
  // two; the softmax sum takes P itself. The lane's tokens 8q + 4g + e (q, e < 4)
  // have their scales in four 16-byte runs; sm_scales(it, h) reads runs 2h and
  // 2h + 1 one phase before sm_exp(8h) uses them. Scales of rows past the
  // visible length are not data: in the tail tile they become 0 (P is 0 there).
  f32x4 psc[2];
  auto sm_scales = [&](int it, int h, auto may_tag) {
    if constexpr (kFp8) {
      constexpr bool kMay = decltype(may_tag)::value;
      const char* sb = lds + (it & (kStages - 1)) * F::bytes + kStage8Scale + 16 * g + 64 * h;
      psc[0] = *reinterpret_cast<const f32x4*>(sb);
      psc[1] = *reinterpret_cast<const f32x4*>(sb + 32);
      const int vlim = t_end - (tile0 + it) * kTok - 4 * g;
      if (kMay && vlim + 4 * g < kTok) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
          if ((16 * h + 8 * (r >> 2) + (r & 3)) >= vlim) psc[r >> 2][r & 3] = 0.f;
      }
    }
  };
  auto sm_exp = [&](int r0) {
#pragma unroll
    for (int r = r0; r < r0 + 8; ++r) {
      xs[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(xs[r], c_log2, -m_ref));
      l_run += xs[r];
      if constexpr (kFp8) xs[r] *= psc[(r - r0) >> 2][r & 3];
    }
  };
  auto sm_pack = [&]() {
#pragma unroll
    for (int r = 0; r < 16; ++r) pb[r >> 3][r & 7] = (__bf16)xs[r];
  };
  auto sm_publish = [&](int it) {
    char* ps = pbuf + ((it & 1) * 8 + wave * 2) * 1024 + lane * 16;
    *reinterpret_cast<bf16x8*>(ps) = pb[0];
    *reinterpret_cast<bf16x8*>(ps + 1024) = pb[1];
  };

#define MLA_FENCE() __builtin_amdgcn_sched_barrier(0)

  // tile `it` without PV (first tile of a pass)
  auto softmax_only = [&](int it, bool& over, auto dma_tag) {
    const f32x16 S = qk(it, dma_tag, std::false_type{});
    sm_scales(it, 0, std::true_type{});
    sm_scale(S, it, std::true_type{});
    sm_localmax();
    sm_ref(over);
    sm_exp(0);
    sm_scales(it, 1, std::true_type{});
    sm_exp(8);
    sm_pack();
    pref_id = load_id(tile0 + min(it + 3, n_tiles - 1));  // for QK(it + 1); clamped into the piece
    sm_publish(it);
    MLA_FENCE();
  };

  // tile `it`: QK(it), then softmax(it) chunks interleaved with PV(it-1),
  // whose first operands QK(it) has already fetched. may_tag: whether the
  // tile can be the piece's partial last one (std::false_type: it is full).
  auto softmax_pv = [&](int it, bool& over, auto dma_tag, auto may_tag) {
    const int ip = it - 1;
    const f32x16 S = qk(it, dma_tag, std::true_type{});
    sm_scale(S, it, may_tag); mm4(0, va[0], pf); va[2] = vfrag(ip, 0, 2); interleave<8>(); MLA_FENCE();
    sm_localmax();         mm4(1, va[1], pf); va[0] = vfrag(ip, 0, 3); sm_scales(it, 0, may_tag); interleave<4>(); MLA_FENCE();
    sm_ref(over);          mm4(2, va[2], pf); va[1] = vfrag(ip, 1, 0); interleave<2>(); MLA_FENCE();
    sm_exp(0);             mm4(3, va[0], pf); interleave<4>(); MLA_FENCE();
    sm_scales(it, 1, may_tag);
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) pf[ht] = pfrag(ip, 1, ht);
    va[2] = vfrag(ip, 1, 1);
    MLA_FENCE();
    sm_exp(8);             mm4(0, va[1], pf); va[0] = vfrag(ip, 1, 2); interleave<4>(); MLA_FENCE();
    sm_pack();             mm4(1, va[2], pf); va[1] = vfrag(ip, 1, 3); interleave<2>(); MLA_FENCE();
    pref_id = load_id(tile0 + min(it + 3, n_tiles - 1));  // for QK(it + 1); clamped into the piece
    sm_publish(it);        mm4(2, va[0], pf); MLA_FENCE();
    // mm4(3, va[1], pf) of PV(ip) runs at the start of the next QK
  };

  // PV(t) alone (the last tile of a pass)
  auto pv_only = [&](int ip) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 pf[4];
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) pf[ht] = pfrag(ip, ks, ht);
#pragma unroll
      for (int cp = 0; cp < 4; ++cp) mm4(cp, vfrag(ip, ks, cp), pf);
    }
  };

  // rows past the visible length may hold anything (even NaN); P is 0 there,
  // so make those rows exactly 0 as well before PV reads them
  auto zero_tail = [&](int it) {
    if constexpr (kFp4) return;  // the dequantized V rows past the end are written as zeros
    const int valid = t_end - (tile0 + it) * kTok;
    if (valid < kTok) {
      char* tb = lds + (it & (kStages - 1)) * F::bytes;
      if constexpr (kFp8) {
        // code rows only: k_R rows feed scores that are masked, and scales are
        // masked where P is formed
        for (int q = tid; q < (kTok - valid) * (kDc / 16); q += kThreads)
          *reinterpret_cast<f32x4*>(tb + valid * kDc + q * 16) = f32x4{};
      } else {
        for (int q = tid; q < (kTok - valid) * (kRowBytes / 16); q += kThreads)
          *reinterpret_cast<f32x4*>(tb + valid * kRowBytes + q * 16) = f32x4{};
      }
    }
  };

  float* const lbuf = reinterpret_cast<float*>(pbuf);   // end-of-pass exchange (reuses the P slots)
  int* const flag = reinterpret_cast<int*>(pbuf + 1024);

  // bf16 query staging (see the piece prologue). Round 0 moves q_abs chunks
  // 0..31 (16-byte chunks, dims 8c..8c+7) of the wave's 32 heads, round 1
  // chunks 32..63 and the q_R rows. Chunk c of head n sits at slot
  // c ^ (n & 15) of the head's 512-byte row, q_R chunk c at c ^ ((n >> 1) & 7)
  // of its 128-byte row, so the MFMA-layout reads (16 heads per 256 bytes of
  // banks) are conflict-free; load j of a round moves heads 2j and 2j + 1.
  constexpr int kQRegion = 20 * 1024;
  static_assert(kScaled || 2 * kStageBytes + 4 * kQRegion <= F::lds, "query staging fits behind stage 1");
  auto q_round = [&](int round) {
    const int ql = lane_here();
    const char* qa_w = reinterpret_cast<const char*>(q_abs + (qbase + wave * 32) * kDc) + round * 512;
    const unsigned reg = (unsigned)(uintptr_t)(lds_void_t*)(lds + 2 * kStageBytes + wave * kQRegion);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      dma16<false>(qa_w + j * 2048, (unsigned)((ql >> 5) * 1024 + (((ql & 31) ^ ((2 * j + (ql >> 5)) & 15)) << 4)),
                   reg + j * 1024);
    if (round == 1) {
      const char* qr_w = reinterpret_cast<const char*>(q_r + (qbase + wave * 32) * kDr);
      const int n = ql >> 3;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dma16<false>(qr_w + j * 1024, (unsigned)(n * 128 + (((ql & 7) ^ (((8 * j + n) >> 1) & 7)) << 4)),
                     reg + 16 * 1024 + j * 1024);
    }
  };
  auto q_read = [&](int round) {
    const int ql = lane_here();
    const int n = ql & 31, gq = ql >> 5;
    const char* qs = lds + 2 * kStageBytes + wave * kQRegion;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
      qf[16 * round + kk] = *reinterpret_cast<const bf16x8*>(qs + n * 512 + (((2 * kk + gq) ^ (n & 15)) << 4));
    if (round == 1) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        qf[32 + kk] = *reinterpret_cast<const bf16x8*>(qs + 16 * 1024 + n * 128 + (((2 * kk + gq) ^ ((n >> 1) & 7)) << 4));
    }
  };

  // ---- piece loop: rows touching [r_lo, r_hi), in order
  while (cb < a.B && cp < r_hi) {
    const int v = cL - a.s_q + ci + 1;          // keys visible to query ci
    const int n_row = v > 0 ? (v + kPage - 1) / kPage : 0;
    const int mid = cp + n_row / 2;  // with S = 1 the row belongs to the range of its middle page
    const bool mine = n_row > 0 && (S > 1 ? cp + n_row > r_lo : (mid >= r_lo && mid < r_hi));
    if (mine) {
      const int pa = S > 1 ? max(r_lo, cp) - cp : 0;
      const int pe = S > 1 ? min(r_hi, cp + n_row) - cp : n_row;
      b = cb;
      i = ci;
      split = S > 1 ? k - cp / W : 0;
      qbase = ((int64_t)b * a.s_q + i) * kH;
      const int t_begin = pa * kPage;
      t_end = min(pe * kPage, v);
      tile0 = t_begin / kTok;
      n_tiles = (t_end - t_begin + kTok - 1) / kTok;
      m_ref = -INFINITY;
      m_seen = -INFINITY;

      // The queries are requested first, so that the page lookups of the first
      // two tiles overlap their transfer; then the two tiles' DMA. Queries and
      // tiles all land before the tile loop (otherwise the compiler re-waits
      // for the queries inside the loop, where the wait would also drain cache
      // DMA).
      // queries: B operand of S^T = K . Q^T; lane (g, lo) holds dims 16kk+8g..+7 of head h_own
      if (n_tiles > 0) {
        const int ql = lane_here();
        const bf16x8* qa = reinterpret_cast<const bf16x8*>(q_abs + (qbase + wave * 32 + (ql & 31)) * kDc);
        const bf16x8* qr = reinterpret_cast<const bf16x8*>(q_r + (qbase + wave * 32 + (ql & 31)) * kDr);
        if constexpr (kScaled) {
          // scaled MFMA m: dims 64m + 16g .. +15 (block 2m) and 64m + 32 + 16g
          // .. +15 (block 2m + 1), held in qf[0..31] until they are split below
#pragma unroll
          for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) qf[4 * m + j] = qa[8 * m + 4 * (j >> 1) + 2 * (ql >> 5) + (j & 1)];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) qf[32 + kk] = qr[2 * kk + (ql >> 5)];
        } else {
          // bf16 cache: the query goes through LDS (stages 2 and 3 and the P
          // slots, idle until tile 2's DMA) so that every load covers whole
          // rows; direct loads in the MFMA layout give each instruction 32-byte
          // pieces of 32 rows 1 KiB apart. Two rounds per wave in a 20 KiB region
          // of its own: q_abs dims 0..255 now, next to the first tiles' DMA; dims
          // 256..511 and q_R once the first half is read.
          q_round(0);
        }
        {
          const DmaTarget d0 = dma_target(tile0, 0);
#pragma unroll
          for (int k = 0; k < F::dma; ++k) dma_piece(d0, k, tile0);
        }
        if (n_tiles > 1) {
          const DmaTarget d1 = dma_target(tile0 + 1, 1);
#pragma unroll
          for (int k = 0; k < F::dma; ++k) dma_piece(d1, k, tile0 + 1);
        }
        if constexpr (!kScaled) {
          if (n_tiles > 1) wait_vmcnt<2 * F::dma>(); else wait_vmcnt<F::dma>();
          q_read(0);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the region is refilled
          q_round(1);
          wait_vmcnt<0>();
          q_read(1);
        } else {
          wait_vmcnt<0>();
        }
        if constexpr (kScaled) {
          // each 32-dim block as hi + lo E4M3 codes; the MFMA operand takes
          // block 2m's 16 dims in bytes 0..15 and block 2m+1's in 16..31, and
          // this lane supplies the scale of block 2m + g
          const int gq = ql >> 5;
          qsh[0] = qsh[1] = qsl[0] = qsl[1] = 0;
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            u32x4 hA, lA, hB, lB;
            int khA, klA, khB, klB;
            split_block_fp8(qf[4 * m], qf[4 * m + 1], hA, lA, khA, klA);
            split_block_fp8(qf[4 * m + 2], qf[4 * m + 3], hB, lB, khB, klB);
            qhl[2 * m] = i32x8{(int)hA[0], (int)hA[1], (int)hA[2], (int)hA[3],
                               (int)hB[0], (int)hB[1], (int)hB[2], (int)hB[3]};
            qhl[2 * m + 1] = i32x8{(int)lA[0], (int)lA[1], (int)lA[2], (int)lA[3],
                                   (int)lB[0], (int)lB[1], (int)lB[2], (int)lB[3]};
            const int kh = gq ? khB : khA, kl = gq ? klB : klA;
            qsh[m >> 2] |= (kh + 127) << (8 * (m & 3));
            qsl[m >> 2] |= (kl + 127) << (8 * (m & 3));
          }
        }
      }

      for (int pass = 0; pass < 2; ++pass) {
        // O^T = 0 through the matrix core, so O is only ever defined by MFMAs
        {
          const bf16x8 z = bf16x8{};
#pragma unroll
          for (int cp = 0; cp < 4; ++cp)
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) O[cp][ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(z, z, f32x16{}, 0, 0, 0);
        }
        l_run = 0.f;
        bool over = false;
#pragma unroll
        for (int k = 0; k < 4; ++k) pf[k] = bf16x8{};
#pragma unroll
        for (int k = 0; k < 3; ++k) va[k] = VFrag{};

        if (n_tiles > 0) {
          // Iteration j issues DMA(j+2) inside its QK phase (only for tiles that
          // exist); stage (j+2)&3 was last read by PV(j-2) in iteration j-1. At
          // the top of iteration it the only loads issued after DMA(it) are those
          // of DMA(it+1).
          if (pass > 0) {  // the first pass's two tiles were issued with the queries
            issue(tile0, 0);
            if (n_tiles > 1) issue(tile0 + 1, 1);
          }
          // tile 0: QK + softmax only
          pref_id = load_id(tile0 + min(2, n_tiles - 1));
          if (n_tiles > 1) wait_vmcnt<F::dma>(); else wait_vmcnt<0>();
          tile_barrier();
          zero_tail(0);
          if (n_tiles > 2)
            softmax_only(0, over, std::true_type{});
          else
            softmax_only(0, over, std::false_type{});
          // steady state: QK(it) + softmax(it) overlapped with PV(it - 1); the
          // last two tiles issue no further DMA
          int it = 1;
          for (; it + 2 < n_tiles; ++it) {  // full tiles: no tail handling
            wait_vmcnt<F::dma>();
            tile_barrier();
            softmax_pv(it, over, std::true_type{}, std::false_type{});
          }
          for (; it < n_tiles; ++it) {
            if (it + 1 < n_tiles) wait_vmcnt<F::dma>(); else wait_vmcnt<0>();
            tile_barrier();
            zero_tail(it);
            softmax_pv(it, over, std::false_type{}, std::true_type{});
          }
          tile_barrier();
          mm4(3, va[1], pf);  // deferred tail of PV(n_tiles - 2)
          pv_only(n_tiles - 1);
        }

        // end of pass: publish per-head sums and whether any score outgrew its reference
        __syncthreads();                        // all P slot reads are done
        if (tid == 0) *flag = 0;
        __syncthreads();
        const float l_tot = l_run + shfl_xor32(l_run);
        if (g == 0) lbuf[h_own] = l_tot;
        if (__any(over) && lane == 0) *flag = 1;
        __syncthreads();
        const bool again = *flag != 0;
        if (!again || pass == 1) break;
        m_ref = m_seen;                          // exact max: a second rescan is impossible
        __syncthreads();                         // everyone has read the flag and lbuf
      }

      // ---- epilogue: normalise, write this split's partial rows and their LSEs.
      // A lane holds 16-byte pieces of one head row, so storing straight from the
      // accumulators would write 32 bytes of 32 different rows per instruction and
      // leave partly written lines behind. Instead each wave stages 32 head rows of
      // its 128-column slice in its own LDS region (the stage ring is idle now) and
      // stores whole 512-byte row slices, two rows per instruction. LDS operations
      // of one wave complete in order, so no barrier is needed between the two.
      constexpr int kEpiStride = 128 * 4 + 16;  // staged row: 512 bytes + 16 of padding against bank conflicts
      char* const ebuf = lds + wave * (32 * kEpiStride);
      const int el = lane_here();
      const int elo = el & 31, eg = el >> 5;
      float inv[4];
      bool empty[4];
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        const float l = lbuf[ht * 32 + elo];
        empty[ht] = !(l > 0.f);
        inv[ht] = empty[ht] ? 0.f : 1.0f / l;
      }
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
        for (int cp = 0; cp < 4; ++cp)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = empty[ht] ? 0.f : O[cp][ht][4 * q + e] * inv[ht];
            *reinterpret_cast<f32x4*>(ebuf + elo * kEpiStride + (32 * cp + 8 * q + 4 * eg) * 4) = v;
          }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = 2 * j + eg;
          const f32x4 v = *reinterpret_cast<const f32x4*>(ebuf + r * kEpiStride + elo * 16);
          float* orow = o_part + ((qbase + ht * 32 + r) * a.num_splits + split) * kDc + wave * 128 + elo * 4;
          *reinterpret_cast<f32x4*>(orow) = v;
        }
        asm volatile("" ::: "memory");
      }
      if (eg == 0) {
        const float l = lbuf[wave * 32 + elo];
        lse_part[(qbase + wave * 32 + elo) * a.num_splits + split] =
            l > 0.f ? (m_ref + __builtin_amdgcn_logf(l)) * 0.69314718055994530942f : -INFINITY;
      }

      // slots past this row's last piece stay empty
      if (S > 1 && cp + n_row <= r_hi) {
        const int rest = S - 1 - split;
        for (int q = tid; q < kH * rest; q += kThreads)
          lse_part[(qbase + q / rest) * S + split + 1 + q % rest] = -INFINITY;
      }
      __syncthreads();  // the next piece reuses the LDS stages and buffers
    }
    cp += n_row;
    if (++ci == a.s_q) {
      ci = 0;
      if (++cb < a.B) cL = clamp_len(seqlens[cb], a.max_pages);
    }
  }
}

template <int kFmt>
constexpr int decode_lds_bytes() { return StageFmt<kFmt>::lds; }
constexpr int kDecodeThreads = kThreads;
constexpr int kDecodeGroups = kScanGroups;

}  // namespace mla
