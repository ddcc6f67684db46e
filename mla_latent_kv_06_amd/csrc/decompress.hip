// Decompressed branch, stage 1: per-head keys and values of every cached
// token (path A of the MLA operator-teardown page, section 4, used for
// chunks above the absorption threshold of section 3):
//     K[b, h, t, d] = sum_c W_UK[h, d, c] c_KV[t, c]
//     V[b, h, t, d] = sum_c W_UV[h, d, c] c_KV[t, c]
// on bf16 MFMA with fp32 accumulation, K rounded once to bf16 and V to fp16
// (V feeds the attention's P.V product, which runs in fp16 for three more
// significant bits at the same matrix-core rate).
//
// Rows t < L_b are written and rows L_b .. the end of that page are
// zero-filled, so the attention stage can read K and V in whole pages.
//
// Workgroup = (head h, sequence b, 256-token tile): the 256 x 256 output tile
// D^T[n, t] with n = the 128 K rows then the 128 V rows of head h. The
// latent columns stream through a ring of 4 LDS stages of 32 columns, filled
// with 16-byte direct-to-LDS loads three chunks ahead (a chunk's MFMAs take
// less time than a memory round trip); the cache rows come through the
// block table. 8 waves, two per SIMD (so one
// wave's loads and LDS traffic overlap the other's MFMAs): wave w computes
// the 128 x 64 part (n half w & 1, token quarter w >> 1) as 4 x 2 tiles of
// v_mfma_f32_32x32x16_bf16 in 128 accumulator registers. Each XCD owns 16
// heads, taken in two groups of 8; within a group the 8 heads of one token
// tile run one after another, so the tile's latent rows (256 KiB) come from
// HBM once and then from the XCD's L2, and the group's 2 MiB of weights stay
// in L2 across tiles.
#include "mla_device.hpp"
#include "prefill.hpp"

namespace mla {

namespace {

constexpr int kDecTok = 256;                    // tokens per workgroup
constexpr int kDecN = 256;                      // output rows: K_h then V_h
constexpr int kDecKc = 32;                      // latent columns per LDS chunk
constexpr int kDecRow = kDecKc * 2;             // 64 bytes per LDS row
constexpr int kDecStage = (kDecN + kDecTok) * kDecRow;  // 32 KiB
constexpr int kDecStages = 4;
constexpr int kDecChunks = kDc / kDecKc;        // 16
constexpr int kDecAhead = 3;                    // chunks in flight ahead of the one computed
constexpr int kDecDmaPerWave = 4;               // 1 KiB loads per wave per chunk

// 16-byte chunk position within a 64-byte LDS row: any 16 consecutive rows
// read at one logical chunk land on 16 distinct 4-bank groups
__device__ __forceinline__ int swz64(int row, int chunk) { return (chunk ^ ((row >> 2) & 3)) << 4; }

// One 16-byte-per-lane direct-to-LDS load: lane l's 16 bytes from
// sbase + voff land at LDS byte address lds_addr + 16 l (lds_addr and sbase
// uniform). Written as asm so that later LDS reads are not treated as
// overlapping it; completion is tracked with explicit vmcnt waits. lds_addr
// is an operand bound to M0, so the compiler writes M0 itself; the s_nop is
// the wait state an LDS-DMA instruction needs after an SALU write of M0.
__device__ __forceinline__ void dma16(const char* sbase, unsigned voff, unsigned lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr)
               : "memory");
}

// Workgroup barrier after this wave's own loads of the chunk have been
// waited for with vmcnt; it does not drain the loads still in flight.
__device__ __forceinline__ void chunk_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace

constexpr int kDecThreads = 512;

__global__ __launch_bounds__(kDecThreads) void decompress_kv_kernel(const char* __restrict__ kv, int64_t num_pages,
                                                            const int32_t* __restrict__ block_table, int max_pages,
                                                            const int32_t* __restrict__ seqlens, int B, int max_len,
                                                            const __bf16* __restrict__ w_uk,
                                                            const __bf16* __restrict__ w_uv, __bf16* __restrict__ k_out,
                                                            _Float16* __restrict__ v_out, int n_tiles, int total,
                                                            int per_xcd) {
  __shared__ __attribute__((aligned(1024))) char lds[kDecStages * kDecStage];
  // blockIdx x runs on XCD x & 7 as its (x >> 3)-th work item
  const int n_bt = B * n_tiles;              // (sequence, token tile) pairs
  const int j = blockIdx.x >> 3;
  const int grp = j / (8 * n_bt);
  const int rem = j - grp * 8 * n_bt;
  const int h = (blockIdx.x & 7) * 16 + grp * 8 + (rem & 7);
  const int bt_idx = rem >> 3;
  const int b = bt_idx / n_tiles;
  const int t0 = (bt_idx - b * n_tiles) * kDecTok;
  (void)total;
  (void)per_xcd;
  int L = clamp_len(seqlens[b], max_pages);
  if (L > max_len) L = max_len;
  if (t0 >= L) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, lo = lane & 31;

  // ---- loader: a stage holds 16 blocks of 1 KiB (16 rows of 64 bytes) of
  // weight rows, then 16 of token rows; wave w fills blocks 2w and 2w + 1 of
  // each. Lane l's slot in a block holds row 16k + l/4 and the logical chunk
  // the swizzle puts at physical chunk l & 3. A weight block lies in W_UK[h]
  // (blocks 0..7) or W_UV[h] (8..15), a token block in one cache page, so each
  // load has a uniform base. Token rows past the sequence read rows of the
  // last page (their outputs are never stored).
  unsigned woff[2], coff[2];
  const char* wbase[2];
  const char* cbase[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int blk = 2 * wave + j;
    const int row = 16 * blk + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    const __bf16* w = blk < 8 ? w_uk + (int64_t)h * kDhc * kDc : w_uv + (int64_t)h * kDhc * kDc;
    wbase[j] = reinterpret_cast<const char*>(w);
    woff[j] = (unsigned)((row & (kDhc - 1)) * kDc * 2 + c * 16);
    const int t_blk = t0 + 16 * blk < L ? t0 + 16 * blk : L - 1;
    const int64_t page = physical_page(block_table, max_pages, b, t_blk >> 6, num_pages);
    cbase[j] = kv + page * kPageBytes;
    coff[j] = (unsigned)(((t0 + row) & (kPage - 1)) * kRowBytes + c * 16);
  }
  const unsigned lds0 = (unsigned)(uintptr_t)(lds_void_t*)lds;
  auto issue = [&](int kc) {
    const unsigned st = lds0 + ((unsigned)kc % (unsigned)kDecStages) * kDecStage;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      dma16(wbase[j], woff[j] + kc * kDecRow, st + (2 * wave + j) * 1024);
      dma16(cbase[j], coff[j] + kc * kDecRow, st + kDecN * kDecRow + (2 * wave + j) * 1024);
    }
  };

  // ---- MFMA tiles of this wave: A = weight rows n, B = token rows t
  const int nb = wave & 1, tq = wave >> 1;
  f32x16 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) acc[mi][ti] = f32x16{};

#pragma unroll
  for (int kc = 0; kc < kDecAhead; ++kc) issue(kc);
  for (int kc = 0; kc < kDecChunks; ++kc) {
    // chunk kc has landed (the chunks after it may still be in flight); after
    // the barrier every wave is done with chunk kc-1, whose stage is refilled
    // with chunk kc + 3
    const int ahead = kDecChunks - 1 - kc < kDecAhead - 1 ? kDecChunks - 1 - kc : kDecAhead - 1;
    if (ahead == 2)
      wait_vmcnt<2 * kDecDmaPerWave>();
    else if (ahead == 1)
      wait_vmcnt<kDecDmaPerWave>();
    else
      wait_vmcnt<0>();
    chunk_barrier();
    if (kc + kDecAhead < kDecChunks) issue(kc + kDecAhead);
    const char* base = lds + ((unsigned)kc % (unsigned)kDecStages) * kDecStage;
#pragma unroll
    for (int ks = 0; ks < kDecKc / 16; ++ks) {
      bf16x8 af[4], bf[2];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int ra = 128 * nb + 32 * m + lo;
        af[m] = *reinterpret_cast<const bf16x8*>(base + ra * kDecRow + swz64(ra, 2 * ks + g));
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int rb = 64 * tq + 32 * m + lo;
        bf[m] = *reinterpret_cast<const bf16x8*>(base + kDecN * kDecRow + rb * kDecRow + swz64(rb, 2 * ks + g));
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
          acc[mi][ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ti], acc[mi][ti], 0, 0, 0);
    }
  }
  __syncthreads();  // every wave is done with the ring before the epilogue reuses it

  // ---- epilogue: the tile goes through LDS so that global writes cover
  // whole 256-byte rows (a (b, h, tile) block of K, and of V, is one
  // contiguous 64 KiB range). Lane owns token 64tq + 32ti + lo and output
  // rows 32mi + 8q + 4g + 0..3; LDS row = 128 values, 16-byte chunk c of
  // token row r stored at chunk c ^ (r & 15).
  {
    char* region = lds + nb * (kDecTok * 256);
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      const int r = 64 * tq + 32 * ti + lo;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& a = acc[mi][ti];
          const int d = 32 * mi + 8 * q + 4 * g;
          char* dst = region + r * 256 + (((d >> 3) ^ (r & 15)) << 4) + (d & 4) * 2;
          if (nb == 0)
            *reinterpret_cast<bf16x4*>(dst) = bf16x4{(__bf16)a[4 * q], (__bf16)a[4 * q + 1], (__bf16)a[4 * q + 2],
                                                     (__bf16)a[4 * q + 3]};
          else
            *reinterpret_cast<f16x4*>(dst) = f16x4{(_Float16)a[4 * q], (_Float16)a[4 * q + 1],
                                                   (_Float16)a[4 * q + 2], (_Float16)a[4 * q + 3]};
        }
    }
  }
  __syncthreads();
  // rows t < L are written, rows L .. (end of L's page) are zero-filled (the
  // attention stage reads whole pages of K and V), later rows are not touched
  const int L_pad = (L + kPage - 1) / kPage * kPage;
  char* kdst = reinterpret_cast<char*>(k_out + (((int64_t)b * kH + h) * max_len + t0) * kDhc);
  char* vdst = reinterpret_cast<char*>(v_out + (((int64_t)b * kH + h) * max_len + t0) * kDhc);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int q = kDecThreads * k + tid, r = q >> 4, c = q & 15;
    const int t = t0 + r;
    if (t >= L_pad) continue;
    const int src = r * 256 + ((c ^ (r & 15)) << 4);
    const bool live = t < L;
    const f32x4 kq = live ? *reinterpret_cast<const f32x4*>(lds + src) : f32x4{};
    const f32x4 vq = live ? *reinterpret_cast<const f32x4*>(lds + kDecTok * 256 + src) : f32x4{};
    // non-temporal: the 4+ GB of K and V would otherwise evict the latent
    // tiles and weights that the next workgroups reuse from L2
    __builtin_nontemporal_store(kq, reinterpret_cast<f32x4*>(kdst + r * 256 + c * 16));
    __builtin_nontemporal_store(vq, reinterpret_cast<f32x4*>(vdst + r * 256 + c * 16));
  }
}

hipError_t launch_decompress_kv(const char* kv, int64_t num_pages, const int32_t* block_table, int max_pages,
                                const int32_t* seqlens, int B, int max_len, const __bf16* w_uk, const __bf16* w_uv,
                                __bf16* k_out, _Float16* v_out, hipStream_t stream) {
  const int n_tiles = (max_len + kDecTok - 1) / kDecTok;
  const int total = kH * B * n_tiles;  // 8 XCDs x 16 heads x (B * n_tiles): every block is a work item
  const int per_xcd = total / 8;
  hipLaunchKernelGGL(decompress_kv_kernel, dim3(total), dim3(kDecThreads), 0, stream, kv, num_pages, block_table,
                     max_pages, seqlens, B, max_len, w_uk, w_uv, k_out, v_out, n_tiles, total, per_xcd);
  return hipGetLastError();
}

}  // namespace mla
