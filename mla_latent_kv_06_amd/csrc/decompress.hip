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
// latent columns are streamed through LDS in chunks of 64 (double-buffered:
// the next chunk's global loads are in flight during the MFMAs of this one);
// the cache rows come through the block table. Wave w computes the 128 x 128
// quarter (n half w & 1, token half w >> 1) as 4 x 4 tiles of
// v_mfma_f32_32x32x16_bf16 in the 256 accumulator registers. Work items are
// dealt over the 8 XCDs in contiguous ranges with the head slowest, so the
// workgroups on one XCD share a head's 256 KiB of weights in its L2.
#include "mla_device.hpp"
#include "prefill.hpp"

namespace mla {

namespace {

constexpr int kDecTok = 256;                    // tokens per workgroup
constexpr int kDecN = 256;                      // output rows: K_h then V_h
constexpr int kDecKc = 64;                      // latent columns per LDS chunk
constexpr int kDecRow = kDecKc * 2;             // 128 bytes per LDS row
constexpr int kDecStage = (kDecN + kDecTok) * kDecRow;  // 64 KiB
constexpr int kDecChunks = kDc / kDecKc;        // 8

// 16-byte chunk position within a 128-byte LDS row: any 16 consecutive rows
// read at one logical chunk land on 16 distinct 4-bank groups
__device__ __forceinline__ int swz128(int row, int chunk) { return (chunk ^ ((row >> 1) & 7)) << 4; }

}  // namespace

__global__ __launch_bounds__(256) void decompress_kv_kernel(const char* __restrict__ kv, int64_t num_pages,
                                                            const int32_t* __restrict__ block_table, int max_pages,
                                                            const int32_t* __restrict__ seqlens, int B, int max_len,
                                                            const __bf16* __restrict__ w_uk,
                                                            const __bf16* __restrict__ w_uv, __bf16* __restrict__ k_out,
                                                            _Float16* __restrict__ v_out, int n_tiles, int total,
                                                            int per_xcd) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kDecStage];
  const int x = blockIdx.x;
  const int id = (x & 7) * per_xcd + (x >> 3);
  if (id >= total) return;
  const int h = id / (B * n_tiles);
  const int rem = id - h * (B * n_tiles);
  const int b = rem / n_tiles;
  const int t0 = (rem - b * n_tiles) * kDecTok;
  int L = clamp_len(seqlens[b], max_pages);
  if (L > max_len) L = max_len;
  if (t0 >= L) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, lo = lane & 31;

  // ---- loader: thread tid moves pieces q = 256k + tid (k = 0..7) of each
  // half: row q >> 3 (0..255), 16-byte chunk q & 7 of the 128-byte slice
  const char* wrow[8];
  const char* crow[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int row = 32 * k + (tid >> 3);
    const __bf16* w = row < kDhc ? w_uk + ((int64_t)h * kDhc + row) * kDc : w_uv + ((int64_t)h * kDhc + row - kDhc) * kDc;
    wrow[k] = reinterpret_cast<const char*>(w) + (tid & 7) * 16;
    int t = t0 + row;
    if (t >= L) t = L - 1;  // rows past the sequence: a valid row whose outputs are never stored
    crow[k] = token_row(kv, block_table, max_pages, b, t, num_pages) + (tid & 7) * 16;
  }
  f32x4 wv[8], cv[8];
  auto load = [&](int kc) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      wv[k] = *reinterpret_cast<const f32x4*>(wrow[k] + kc * kDecRow);
      cv[k] = *reinterpret_cast<const f32x4*>(crow[k] + kc * kDecRow);
    }
  };
  auto store = [&](int stage) {
    char* base = lds + stage * kDecStage;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int row = 32 * k + (tid >> 3);
      const int off = row * kDecRow + swz128(row, tid & 7);
      *reinterpret_cast<f32x4*>(base + off) = wv[k];
      *reinterpret_cast<f32x4*>(base + kDecN * kDecRow + off) = cv[k];
    }
  };

  // ---- MFMA tiles of this wave: A = weight rows n, B = token rows t
  const int nb = wave & 1, tb = wave >> 1;
  f32x16 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) acc[mi][ti] = f32x16{};

  load(0);
  store(0);
  __syncthreads();
  for (int kc = 0; kc < kDecChunks; ++kc) {
    if (kc + 1 < kDecChunks) load(kc + 1);
    const char* base = lds + (kc & 1) * kDecStage;
#pragma unroll
    for (int ks = 0; ks < kDecKc / 16; ++ks) {
      bf16x8 af[4], bf[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int ra = 128 * nb + 32 * m + lo;
        const int rb = 128 * tb + 32 * m + lo;
        af[m] = *reinterpret_cast<const bf16x8*>(base + ra * kDecRow + swz128(ra, 2 * ks + g));
        bf[m] = *reinterpret_cast<const bf16x8*>(base + kDecN * kDecRow + rb * kDecRow + swz128(rb, 2 * ks + g));
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
          acc[mi][ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[ti], acc[mi][ti], 0, 0, 0);
    }
    if (kc + 1 < kDecChunks) store((kc + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: the tile goes through LDS so that global writes cover
  // whole 256-byte rows (a (b, h, tile) block of K, and of V, is one
  // contiguous 64 KiB range). Lane owns token 128tb + 32ti + lo and output
  // rows 32mi + 8q + 4g + 0..3; LDS row = 128 values, 16-byte chunk c of
  // token row r stored at chunk c ^ (r & 15).
  {
    char* region = lds + nb * (kDecTok * 256);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      const int r = 128 * tb + 32 * ti + lo;
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
  for (int k = 0; k < 16; ++k) {
    const int q = 256 * k + tid, r = q >> 4, c = q & 15;
    const int t = t0 + r;
    if (t >= L_pad) continue;
    const int src = r * 256 + ((c ^ (r & 15)) << 4);
    const bool live = t < L;
    *reinterpret_cast<f32x4*>(kdst + r * 256 + c * 16) = live ? *reinterpret_cast<const f32x4*>(lds + src) : f32x4{};
    *reinterpret_cast<f32x4*>(vdst + r * 256 + c * 16) =
        live ? *reinterpret_cast<const f32x4*>(lds + kDecTok * 256 + src) : f32x4{};
  }
}

hipError_t launch_decompress_kv(const char* kv, int64_t num_pages, const int32_t* block_table, int max_pages,
                                const int32_t* seqlens, int B, int max_len, const __bf16* w_uk, const __bf16* w_uv,
                                __bf16* k_out, _Float16* v_out, hipStream_t stream) {
  const int n_tiles = (max_len + kDecTok - 1) / kDecTok;
  const int total = kH * B * n_tiles;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL(decompress_kv_kernel, dim3(per_xcd * 8), dim3(256), 0, stream, kv, num_pages, block_table,
                     max_pages, seqlens, B, max_len, w_uk, w_uv, k_out, v_out, n_tiles, total, per_xcd);
  return hipGetLastError();
}

}  // namespace mla
