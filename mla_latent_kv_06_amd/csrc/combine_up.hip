// Stage 2 of the split scan fused with the per-head up-projection: the split
// partials of a row are merged by their log-sum-exp (KV-split reduction of the
// K3 time-share study, "Inside the blocks") and the merged latent row is
// multiplied by W_UV[h] (absorbed output side of the MLA operator-teardown
// page, section 4) in one pass, so the fp32 o_lat tile never leaves LDS.
//
// Workgroup = (head h, tile of R = 8 or 16 query rows t), 8 waves:
//   * merge, R = 16: wave w merges rows t0 + w and t0 + w + 8 as
//     combine_kernel does (split weights by readlane, the loads of up to 24
//     splits in flight, or 4 when rows have at most 16 splits so that two
//     workgroups fit on a CU; empty splits never read) into the LDS tile;
//   * merge, R = 8 (at most 32 rows in all: few rows, latency-bound): the
//     rows of the tile share the 8 waves (8, 4, 2 or 1 waves per row for
//     1, 2, 3-4 or 5-8 rows), each wave merging a contiguous range of the
//     row's splits with up to 16 in flight; the waves' sums are added in LDS
//     in wave order, so the result does not depend on timing. A single row's
//     32 splits thus take one round of loads instead of two in one wave.
//     Lane l owns latent columns 4l..4l+3 and 256+4l..+3, so every load
//     instruction covers 1 KiB of contiguous memory; the split LSEs are read
//     first, on their own;
//   * W_UV[h] fragments (output rows 16w..16w+15, all 512 latent columns) are
//     requested with R = 8 right after the row's LSE load, so their transfer
//     overlaps the LSE round trip (long workload: 20.7 -> 19.3 us), with
//     R = 16 after both rows' merge loads, so the merge waits only on its own
//     data and the weight loads overlap it, the LDS writes and the barrier. The workgroups of one head are 128 apart in the grid, hence on
//     the same XCD, and share W_UV[h] through its L2;
//   * up-projection: out^T[d, t] = sum_c W_UV[h][d][c] o_lat[t][c] on
//     v_mfma_f32_16x16x32_bf16 (16 rows d x 16 columns t, of which the tile's
//     R are real, x 32 latent columns c), the fp32 o_lat fed as a bf16 high
//     part plus a bf16 remainder (two MFMAs per step, ~16 significant bits).
//     Each merged row is split into the two parts once, as it is written to
//     LDS, so the 8 waves read bf16 operands instead of each converting the
//     whole tile again. The partials are loaded non-temporally (each is read
//     once), which keeps the shared W_UV fragments in L2.
// R = 8 spreads few rows over more workgroups; R = 16 halves the W_UV reads
// per row where there are rows enough to fill the chip. With more 16-row tiles
// than kRowTileGroups per head, a workgroup takes every kRowTileGroups-th tile
// of its head and keeps W_UV[h]'s fragments in registers across them; with one
// split per row the merge is the identity and up_one_split_kernel (below)
// streams the partials instead.
// In k-step ks, lane quad q holds latent columns 32ks + 8q .. +7 of both
// operands, so one instruction reads 64 contiguous bytes of each W_UV row.
#include "mla_device.hpp"
#include "decode.hpp"

namespace mla {

namespace {

constexpr int kTileCols = 16;     // MFMA columns: the tile's rows, then zero rows
constexpr int kSmallTileMaxRows = 32;  // T up to this: 8-row tiles, else 16-row tiles
constexpr int kTileStride = kDc + 8;  // bf16 per tile row; the pad spreads the 16 rows of an MFMA read over the banks
constexpr int kMergeChunk = 24;       // splits whose loads are in flight together (16-row tiles)
constexpr int kFewChunk = 4;          // the same with few splits per row (see launch_combine_up)
constexpr int kFewSplits16 = 16;      // 16-row tiles use kFewChunk up to this many splits
// 16-row tiles with 2..16 splits: at most this many workgroups per head, each
// looping over tiles (1024 rows, one split: 165 us against 178 us with a
// workgroup per tile, which rereads the head's 128 KiB of W_UV for 16 rows)
constexpr int kRowTileGroups = 4;

typedef float f32x4v __attribute__((ext_vector_type(4)));

}  // namespace

// The merge of one row: the split weights w_s = exp(lse_s - L) of the row's
// LSE L (empty splits, lse = -inf, weigh 0 and are never read), then
// sum_s w_s o_s over the splits [sa, sb) into a0 (columns 4l..4l+3) and a1
// (columns 256 + 4l..+3). l0 = lse of split `lane` (-inf past the end).
// before_wait runs once, right after the first loads of
// partials are issued (the W_UV fragments are requested there, so the merge
// waits only on its own data).
template <int kChunk, class F>
__device__ __forceinline__ void merge_range(const float* __restrict__ lp, const float* __restrict__ op, int num_splits,
                                            float l0, float L, int sa, int sb, int lane, f32x4v& a0, f32x4v& a1,
                                            F&& before_wait) {
  f32x4v v0[kChunk], v1[kChunk];
  bool first = true;
  for (int b0 = sa & ~63; b0 < sb; b0 += 64) {  // blocks of 64 splits: lane k holds the weight of b0 + k
    const float lb = b0 == 0 ? l0 : (b0 + lane < num_splits ? lp[b0 + lane] : -INFINITY);
    const float wl = expf(lb - L);  // 0 when lse = -inf
    auto weight = [&](int s) {
      return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s - b0));
    };
    const int e = min(b0 + 64, sb);
    for (int s0 = max(b0, sa); s0 < e; s0 += kChunk) {
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        if (s0 + k < e && weight(s0 + k) > 0.f) {
          // partials are read once: non-temporal, so they do not push W_UV out of L2
          v0[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(op + (int64_t)(s0 + k) * kDc));
          v1[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(op + (int64_t)(s0 + k) * kDc + kDc / 2));
        }
      }
      if (first) {
        before_wait();
        first = false;
      }
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        if (s0 + k < e) {
          const float w = weight(s0 + k);
          if (w > 0.f) {
            a0 += w * v0[k];
            a1 += w * v1[k];
          }
        }
      }
    }
  }
  if (first) before_wait();
}

// The row's LSE statistics: l0 = lse of split `lane`, M = max, L = M + log sum exp
// (-inf when every split is empty). after_load runs right after the first LSE
// load is issued: loads requested there overlap its round trip, and the wait
// for the LSE (vector loads complete in order) does not wait for them.
template <class G = void (*)()>
__device__ __forceinline__ void row_lse(const float* __restrict__ lp, int num_splits, int lane, float& l0, float& L,
                                        G&& after_load = [] {}) {
  l0 = lane < num_splits ? lp[lane] : -INFINITY;
  after_load();
  float M = l0;
  for (int s = lane + 64; s < num_splits; s += 64) M = fmaxf(M, lp[s]);
  M = wave_max_dpp(M);
  L = -INFINITY;
  if (M != -INFINITY) {
    float tot = expf(l0 - M);
    for (int s = lane + 64; s < num_splits; s += 64) tot += expf(lp[s] - M);
    L = M + logf(wave_sum_dpp(tot));
  }
}

template <int kRows, int kChunk, bool kLoop = false>
__global__ __launch_bounds__(512) void combine_up_kernel(const float* __restrict__ o_part,
                                                         const float* __restrict__ lse_part,
                                                         const __bf16* __restrict__ w_uv, int T, int num_splits,
                                                         __bf16* __restrict__ out, float* __restrict__ lse_out) {
  static_assert(kRows == 8 || kRows == 16, "one or two rows per wave");
  // the merged o_lat tile as the MFMA's B operand: bf16 high parts (tile[0]) and
  // bf16 remainders (tile[1]), split once as each row is merged
  __shared__ __attribute__((aligned(16))) __bf16 tile[2][kTileCols * kTileStride];
  auto put4 = [&](int row, int col, const f32x4v& v) {
    bf16x4 hi, lw;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hi[j] = (__bf16)v[j];
      lw[j] = (__bf16)(v[j] - (float)hi[j]);
    }
    *reinterpret_cast<bf16x4*>(&tile[0][row * kTileStride + col]) = hi;
    *reinterpret_cast<bf16x4*>(&tile[1][row * kTileStride + col]) = lw;
  };
  // per-wave sums of a row merged by several waves: [wave][column half][lane]
  __shared__ f32x4v wsum[kRows == 8 ? 8 : 1][2][64];
  const int h = blockIdx.x % kH;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r = lane & 15;

  // W_UV[h] rows d = 16w + r, columns 32ks + 8q .. +7 for k-steps ks = 0..15,
  // requested once the merge's own loads are under way
  bf16x8 a[16];
  auto load_w = [&]() {
    const bf16x8* wp = reinterpret_cast<const bf16x8*>(w_uv + ((int64_t)h * kDhc + 16 * wave + r) * kDc + 8 * q);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) a[ks] = wp[4 * ks];
  };

  // Workgroup x handles row tiles x / kH, x / kH + gridDim.x / kH, ... of head
  // x mod kH, holding W_UV[h]'s fragments in registers from its first tile on
  // (a workgroup per tile would read the head's 128 KiB of W_UV for 16 rows).
  bool first = true;
  for (int t0 = (blockIdx.x / kH) * kRows; t0 < T; t0 += (gridDim.x / kH) * kRows) {
    const int rows_here = min(kRows, T - t0);
    if (!first) __syncthreads();  // every wave has read the previous tile
    if constexpr (kRows == 16) {
      // ---- merge rows t0 + w and t0 + w + 8 into LDS rows w and w + 8; zeros
      // past the end, never stored. W_UV is requested after both rows' loads.
      for (int rr = wave; rr < kTileCols; rr += 8) {
        f32x4v a0 = f32x4v{}, a1 = f32x4v{};
        if (rr < rows_here) {
          const int64_t row = (int64_t)(t0 + rr) * kH + h;
          const float* lp = lse_part + row * num_splits;
          float l0, L;
          row_lse(lp, num_splits, lane, l0, L);
          if (L != -INFINITY)
            merge_range<kChunk>(lp, o_part + row * num_splits * kDc + 4 * lane, num_splits, l0, L, 0, num_splits,
                                     lane, a0, a1, [] {});
          if (lane == 0) lse_out[row] = L;
        }
        put4(rr, 4 * lane, a0);
        put4(rr, kDc / 2 + 4 * lane, a1);
      }
      if (first) load_w();
    } else {
      // ---- few rows: a row's splits are dealt to wpr waves (8 / 4 / 2 / 1 for
      // 1 / 2 / 3-4 / 5-8 rows), each wave merging a contiguous range; the wave
      // sums are then added in wave order, so the result does not depend on timing
      const int wpr_log = rows_here == 1 ? 3 : rows_here == 2 ? 2 : rows_here <= 4 ? 1 : 0;
      const int rr = wave >> wpr_log, j = wave & ((1 << wpr_log) - 1);
      f32x4v a0 = f32x4v{}, a1 = f32x4v{};
      bool requested = false;
      if (rr < rows_here) {
        const int64_t row = (int64_t)(t0 + rr) * kH + h;
        const float* lp = lse_part + row * num_splits;
        float l0, L;
        row_lse(lp, num_splits, lane, l0, L, [&] {
          if (first) load_w();
          requested = true;
        });
        if (L != -INFINITY) {
          const int cnt = (num_splits + (1 << wpr_log) - 1) >> wpr_log;
          const int sa = min(num_splits, j * cnt), sb = min(num_splits, sa + cnt);
          merge_range<kChunk>(lp, o_part + row * num_splits * kDc + 4 * lane, num_splits, l0, L, sa, sb, lane, a0, a1, [&] {
            if (!requested && first) load_w();
            requested = true;
          });
        }
        if (j == 0 && lane == 0) lse_out[row] = L;
      }
      if (!requested && first) load_w();
      if (wpr_log == 0) {
        // one wave per row: rows w and w + 8 (zeros past the tile's rows)
        put4(wave, 4 * lane, a0);
        put4(wave, kDc / 2 + 4 * lane, a1);
        put4(wave + 8, 4 * lane, f32x4v{});
        put4(wave + 8, kDc / 2 + 4 * lane, f32x4v{});
      } else {
        wsum[wave][0][lane] = a0;
        wsum[wave][1][lane] = a1;
        __syncthreads();
        // 16 rows x 128 column quads, four per thread
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = tid + 512 * i, row = e >> 7, c4 = e & 127;
          f32x4v v = f32x4v{};
          if (row < rows_here) {
            for (int jj = 0; jj < (1 << wpr_log); ++jj) v += wsum[(row << wpr_log) + jj][c4 >> 6][c4 & 63];
          }
          put4(row, 4 * c4, v);
        }
      }
    }

    __syncthreads();

    // ---- up-projection of the tile: D[d][t], d = 16w + 4q + i, t = t0 + r
    f32x4 acc = f32x4{};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const int off = r * kTileStride + 32 * ks + 8 * q;
      const bf16x8 hi = *reinterpret_cast<const bf16x8*>(&tile[0][off]);
      const bf16x8 lw = *reinterpret_cast<const bf16x8*>(&tile[1][off]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], hi, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], lw, acc, 0, 0, 0);
    }
    const int t = t0 + r;
    if (r < kRows && t < T) {
      const bf16x4 o = {(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3]};
      *reinterpret_cast<bf16x4*>(out + ((int64_t)t * kH + h) * kDhc + 16 * wave + 4 * q) = o;
    }
    if constexpr (!kLoop) break;
    first = false;
  }
}

// ---- one split per row (a chunk of query rows whose pieces were not cut):
// the merge is the identity (weight exp(lse - lse) = 1, LSE unchanged), so
// the kernel streams the partial rows through LDS and only up-projects.
// Workgroup = (head h, every kOneSplitGroups-th 16-row tile), W_UV[h]'s
// fragments in registers for all its tiles. Tiles reach LDS through
// direct-to-LDS loads (each load instruction moves 1 KiB of one partial row;
// each wave also moves the tile's 16 LSEs) into a ring of two stages, so one
// tile is in flight while the previous one is split and multiplied; two
// workgroups share a CU and fill each other's gaps. A tile is read into
// registers, split into bf16 high parts and remainders, and written back over
// its own stage as the MFMA operand, then multiplied as in combine_up_kernel.
// At 1024 rows: 69 us, where one workgroup per 16-row tile (combine_up_kernel)
// took 178 us and a ring of four stages with one workgroup per CU 76 us.
namespace {

constexpr int kOneSplitGroups = 4;                      // workgroups per head: 512 in all, two per CU
constexpr int kOneSplitRing = 2;                        // LDS stages per workgroup
constexpr int kOneSplitTileBytes = 16 * kDc * 4;        // 16 fp32 partial rows
constexpr int kOneSplitStageBytes = kOneSplitTileBytes + 8 * 64 * 4;  // + each wave's copy of the 16 LSEs (x4)
constexpr int kSplitTileBytes = 2 * kTileCols * kTileStride * 2;      // bf16 high parts, then remainders
static_assert(kSplitTileBytes <= kOneSplitStageBytes, "the split tile fits in its stage");
static_assert(kOneSplitRing >= 2 && kOneSplitRing <= 4, "at most two tiles issued after the one waited for");
static_assert(2 * kOneSplitRing * kOneSplitStageBytes <= 160 * 1024, "two workgroups per CU");

// lane l's 16 (4) bytes from sbase + voff land at LDS byte address
// lds_addr + 16 l (4 l); lds_addr is bound to M0, and the s_nop is the wait
// state an LDS-DMA instruction needs after an SALU write of M0. Completion is
// tracked with explicit vmcnt waits.
__device__ __forceinline__ void lds_dma_x4(const void* sbase, unsigned voff, unsigned lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}
__device__ __forceinline__ void lds_dma_x1(const void* sbase, unsigned voff, unsigned lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}
__device__ __forceinline__ unsigned lds_address(const void* p) {
  return (unsigned)(uintptr_t)(const lds_void_t*)p;
}
// all LDS operations of this wave are done, then the workgroup barrier; unlike
// __syncthreads() it leaves the tile loads in flight
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace

__global__ __launch_bounds__(512) void up_one_split_kernel(const float* __restrict__ o_part,
                                                           const float* __restrict__ lse_part,
                                                           const __bf16* __restrict__ w_uv, int T,
                                                           __bf16* __restrict__ out, float* __restrict__ lse_out) {
  __shared__ __attribute__((aligned(16))) char ring[kOneSplitRing * kOneSplitStageBytes];
  const int h = blockIdx.x % kH, grp = blockIdx.x / kH, groups = gridDim.x / kH;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r = lane & 15;
  const int n_tiles = (T + 15) / 16;
  const int mine = n_tiles > grp ? (n_tiles - grp + groups - 1) / groups : 0;  // this workgroup's tiles

  // tile i of this workgroup (rows t0 .. t0 + 15) into stage i % kOneSplitRing:
  // load k moves chunk c = 512k + tid (row c >> 7, 16-byte column chunk
  // c & 127); rows past T re-read row T - 1 and are never used
  auto issue = [&](int i) {
    const int t0 = (grp + i * groups) * 16;
    const int last = min(16, T - t0) - 1;
    char* st = ring + (i % kOneSplitRing) * kOneSplitStageBytes;
    const float* base = o_part + ((int64_t)t0 * kH + h) * kDc;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = 512 * k + tid;
      lds_dma_x4(base, (unsigned)(min(c >> 7, last) * (kH * kDc * 4) + (c & 127) * 16),
                 lds_address(st + (512 * k + 64 * wave) * 16));
    }
    lds_dma_x1(lse_part + (int64_t)t0 * kH + h, (unsigned)(min(lane & 15, last) * (kH * 4)),
               lds_address(st + kOneSplitTileBytes + wave * 256));
  };
  constexpr int kPerTile = 5;  // load instructions per wave and tile

  bf16x8 a[16];  // W_UV[h] rows d = 16w + r, columns 32ks + 8q .. +7
  {
    const bf16x8* wp = reinterpret_cast<const bf16x8*>(w_uv + ((int64_t)h * kDhc + 16 * wave + r) * kDc + 8 * q);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) a[ks] = wp[4 * ks];
  }
#pragma unroll
  for (int i = 0; i < kOneSplitRing - 1; ++i)
    if (i < mine) issue(i);

  for (int i = 0; i < mine; ++i) {
    // tile i has landed once at most the loads issued after it (up to
    // kOneSplitRing - 2 tiles, and the stores of earlier tiles) are
    // outstanding; waiting for fewer is also safe
    const int after = min(kOneSplitRing - 2, mine - 1 - i);  // tiles issued after tile i
    if (after >= 2)
      wait_vmcnt<2 * kPerTile>();
    else if (after == 1)
      wait_vmcnt<kPerTile>();
    else
      wait_vmcnt<0>();
    // every wave's loads of tile i are in LDS, and every wave has finished the
    // MFMAs of tile i - 1, whose stage is refilled now
    lds_barrier();
    if (i + kOneSplitRing - 1 < mine) issue(i + kOneSplitRing - 1);

    const int t0 = (grp + i * groups) * 16;
    const int rows_here = min(16, T - t0);
    char* const st = ring + (i % kOneSplitRing) * kOneSplitStageBytes;
    __bf16* const hi_t = reinterpret_cast<__bf16*>(st);
    __bf16* const lo_t = hi_t + kTileCols * kTileStride;
    // thread: row tid >> 5, columns 4 cg + 128 j .. +3 (j < 4), cg = tid & 31
    const int row = tid >> 5, cg = tid & 31;
    f32x4v v[4];
    const float l = *reinterpret_cast<const float*>(st + kOneSplitTileBytes + wave * 256 + row * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const f32x4v*>(st + row * (kDc * 4) + (4 * cg + 128 * j) * 4);
    if (row < rows_here && cg == 0) lse_out[(int64_t)(t0 + row) * kH + h] = l;
    lds_barrier();  // the whole stage is in registers: its bytes take the split tile
    const bool live = row < rows_here && l != -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // 0 + v: a merged row starts from +0, so -0 becomes +0 here as well
      const f32x4v m = live ? f32x4v{} + v[j] : f32x4v{};
      bf16x4 hi, lw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = (__bf16)m[e];
        lw[e] = (__bf16)(m[e] - (float)hi[e]);
      }
      *reinterpret_cast<bf16x4*>(&hi_t[row * kTileStride + 4 * cg + 128 * j]) = hi;
      *reinterpret_cast<bf16x4*>(&lo_t[row * kTileStride + 4 * cg + 128 * j]) = lw;
    }
    lds_barrier();

    f32x4 acc = f32x4{};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const int off = r * kTileStride + 32 * ks + 8 * q;
      const bf16x8 hi = *reinterpret_cast<const bf16x8*>(&hi_t[off]);
      const bf16x8 lw = *reinterpret_cast<const bf16x8*>(&lo_t[off]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], hi, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], lw, acc, 0, 0, 0);
    }
    if (r < rows_here) {
      const bf16x4 o = {(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3]};
      *reinterpret_cast<bf16x4*>(out + ((int64_t)(t0 + r) * kH + h) * kDhc + 16 * wave + 4 * q) = o;
    }
  }
}

hipError_t launch_combine_up(const float* o_part, const float* lse_part, const __bf16* w_uv, int T, int num_splits,
                             __bf16* out, float* lse, hipStream_t stream) {
  // With few splits per row the merge keeps loads of only kFewChunk splits in
  // flight per wave: the 16-row kernel then needs 128 registers, so two
  // 512-thread workgroups share a CU (one with the deep chunk: 222 registers).
  // The 8-row kernel holds W_UV's fragments through the merge and stays at one
  // workgroup per CU either way, so it takes the short chunk only where that
  // costs no extra round of loads.
  if (T <= kSmallTileMaxRows) {
    const dim3 grid(kH * ((T + 7) / 8));
    if (num_splits <= kFewChunk)
      hipLaunchKernelGGL((combine_up_kernel<8, kFewChunk>), grid, dim3(512), 0, stream, o_part, lse_part, w_uv, T,
                         num_splits, out, lse);
    else
      hipLaunchKernelGGL((combine_up_kernel<8, 16>), grid, dim3(512), 0, stream, o_part, lse_part, w_uv, T, num_splits,
                         out, lse);
  } else {
    const int tiles = (T + 15) / 16;
    if (tiles > kRowTileGroups && num_splits == 1)
      hipLaunchKernelGGL(up_one_split_kernel, dim3(kH * kOneSplitGroups), dim3(512), 0, stream, o_part, lse_part,
                         w_uv, T, out, lse);
    else if (tiles > kRowTileGroups && num_splits <= kFewSplits16)
      hipLaunchKernelGGL((combine_up_kernel<16, kFewChunk, true>), dim3(kH * kRowTileGroups), dim3(512), 0, stream,
                         o_part, lse_part, w_uv, T, num_splits, out, lse);
    else if (num_splits <= kFewSplits16)
      hipLaunchKernelGGL((combine_up_kernel<16, kFewChunk>), dim3(kH * tiles), dim3(512), 0, stream, o_part, lse_part,
                         w_uv, T, num_splits, out, lse);
    else
      hipLaunchKernelGGL((combine_up_kernel<16, kMergeChunk>), dim3(kH * tiles), dim3(512), 0, stream, o_part,
                         lse_part, w_uv, T, num_splits, out, lse);
  }
  return hipGetLastError();
}

}  // namespace mla
