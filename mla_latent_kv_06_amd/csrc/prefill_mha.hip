// Decompressed branch, stage 2: causal multi-head attention over the per-head
// keys and values of stage 1 (path A of the MLA operator-teardown page,
// section 4; used for chunks above the absorption threshold, section 3):
//     s[t] = (q_c[i, h] . K[b, h, t] + q_R[i, h] . k_R[t]) * scale
//     out[i, h] = softmax(s over t <= L_b - s_q + i) . V[b, h, :]
// with 192-dim scores (128 content + the 64-dim RoPE key shared by all
// heads, read from the paged cache) and 128-dim values.
//
// Workgroup = (sequence b, head h, block of 128 queries), 4 waves of 32
// queries. The keys stream in tiles of 64 (one page) through two LDS stages
// (the next tile's global loads are in flight during this tile's MFMAs):
//   * QK: S^T[32 tokens, 32 queries] per token half on v_mfma_f32_32x32x16_bf16,
//     A = key rows from LDS, B = the wave's queries held in 48 VGPRs; a lane
//     owns one query and 16 of each 32 tokens;
//   * softmax in the exp2 domain with a per-query reference max that is only
//     raised (rescaling the accumulator) when a tile's max exceeds it by more
//     than 8, so P <= 2^8;
//   * PV: O^T[128 dims, 32 queries] += V^T . P^T on v_mfma_f32_32x32x16_f16
//     (fp16 V from stage 1 and fp16 P <= 2^8: three more significant bits
//     than bf16 at the same rate), P^T taken straight from the lane's own
//     scores (the reduction over tokens is permuted to the score layout) and
//     V^T read with transposed LDS reads in the same order.
#include "mla_device.hpp"
#include "prefill.hpp"

namespace mla {

namespace {

constexpr int kMhaQ = 128;       // queries per workgroup
constexpr int kMhaTok = 64;      // keys per tile (one page)
constexpr int kKRow = 256;       // bytes of a content-key or value row
constexpr int kRRow = 128;       // bytes of a RoPE-key row
constexpr int kMhaStage = kMhaTok * (2 * kKRow + kRRow);  // 40 KiB: K, V, k_R
constexpr float kRescaleSlack = 8.f;                      // log2 units

// 16-byte chunk positions: key rows (QK reads 16 consecutive rows at one
// chunk), value rows (transposed reads of 4 rows x 4 chunks), RoPE rows
__device__ __forceinline__ int swz_k(int row, int chunk) { return (chunk ^ (row & 15)) << 4; }
__device__ __forceinline__ int swz_v(int row, int chunk) { return (chunk ^ ((row & 3) << 2)) << 4; }
__device__ __forceinline__ int swz_r(int row, int chunk) { return (chunk ^ ((row >> 1) & 7)) << 4; }

__device__ __forceinline__ f16x8 cat8(i16x4 a, i16x4 b) {
  const f16x4 x = __builtin_bit_cast(f16x4, a), y = __builtin_bit_cast(f16x4, b);
  return f16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

}  // namespace

__global__ __launch_bounds__(256) void prefill_mha_kernel(const __bf16* __restrict__ q_c, const __bf16* __restrict__ q_r,
                                                          const __bf16* __restrict__ k_nope,
                                                          const _Float16* __restrict__ v_in, int max_len,
                                                          const char* __restrict__ kv, int64_t num_pages,
                                                          const int32_t* __restrict__ block_table, int max_pages,
                                                          const int32_t* __restrict__ seqlens, int s_q, float scale_log2,
                                                          __bf16* __restrict__ out, float* __restrict__ lse,
                                                          int n_qb, int B, int total, int per_xcd) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kMhaStage];
  const int x = blockIdx.x;
  const int id = (x & 7) * per_xcd + (x >> 3);
  if (id >= total) return;
  const int qb = id % n_qb;
  const int bh = id / n_qb;
  const int h = bh % kH;
  const int b = bh / kH;
  (void)B;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, lo = lane & 31;

  int L = clamp_len(seqlens[b], max_pages);
  if (L > max_len) L = max_len;
  const int i0 = qb * kMhaQ;
  const int i_last = min(i0 + kMhaQ, s_q) - 1;
  const int kv_end = max(0, L - s_q + i_last + 1);       // keys the block's last query sees
  const int n_first = L - s_q + i0 + 1;                  // keys the block's first query sees
  const int n_tiles = (kv_end + kMhaTok - 1) / kMhaTok;

  // this lane's query and the number of keys it sees
  const int iq = i0 + 32 * wave + lo;
  const bool q_live = iq < s_q;
  const int n_vis = q_live ? L - s_q + iq + 1 : 0;

  // ---- queries: B operand, dims 16ks + 8g .. +7 (content 0..127, RoPE 128..191)
  bf16x8 qf[12];
  {
    const int64_t row = ((int64_t)b * s_q + (q_live ? iq : 0)) * kH + h;
    const bf16x8* qc = reinterpret_cast<const bf16x8*>(q_c + row * kDhc);
    const bf16x8* qr = reinterpret_cast<const bf16x8*>(q_r + row * kDr);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = q_live ? qc[2 * ks + g] : bf16x8{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[8 + ks] = q_live ? qr[2 * ks + g] : bf16x8{};
  }

  // ---- loader: per tile 64 rows of K and V (1024 pieces each, 4 per thread)
  // and of k_R (512 pieces, 2 per thread)
  const char* kbase = reinterpret_cast<const char*>(k_nope + ((int64_t)b * kH + h) * max_len * kDhc);
  const char* vbase = reinterpret_cast<const char*>(v_in + ((int64_t)b * kH + h) * max_len * kDhc);
  f32x4 kvv[4], vvv[4], rvv[2];
  auto load = [&](int it) {
    const int t0 = it * kMhaTok;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = 256 * k + tid, row = q >> 4, ch = q & 15;
      kvv[k] = *reinterpret_cast<const f32x4*>(kbase + (int64_t)(t0 + row) * kKRow + ch * 16);
      vvv[k] = *reinterpret_cast<const f32x4*>(vbase + (int64_t)(t0 + row) * kKRow + ch * 16);
    }
    const int64_t page = physical_page(block_table, max_pages, b, it, num_pages);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int q = 256 * k + tid, row = q >> 3, ch = q & 7;
      rvv[k] = *reinterpret_cast<const f32x4*>(kv + page * kPageBytes + (int64_t)row * kRowBytes + kDc * 2 + ch * 16);
    }
  };
  auto store = [&](int it) {
    char* st = lds + (it & 1) * kMhaStage;
    const int valid = L - it * kMhaTok;  // value rows past the sequence become zeros
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = 256 * k + tid, row = q >> 4, ch = q & 15;
      *reinterpret_cast<f32x4*>(st + row * kKRow + swz_k(row, ch)) = kvv[k];
      *reinterpret_cast<f32x4*>(st + kMhaTok * kKRow + row * kKRow + swz_v(row, ch)) =
          row < valid ? vvv[k] : f32x4{};
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int q = 256 * k + tid, row = q >> 3, ch = q & 7;
      *reinterpret_cast<f32x4*>(st + 2 * kMhaTok * kKRow + row * kRRow + swz_r(row, ch)) = rvv[k];
    }
  };

  // ---- V^T operand offsets: group G = lane >> 4, ii = lane & 15 reads token
  // row 4(G >> 1) + (ii >> 2) (+8 for the second half, +16 per k-step, +32 per
  // token half) and 4 columns 16(G & 1) + 4(ii & 3) of a 32-column tile
  const int Gq = lane >> 4, ii = lane & 15;
  const int t_lane = 4 * (Gq >> 1) + (ii >> 2);
  const int jl = 2 * (Gq & 1) + ((ii & 3) >> 1);
  auto vfrag = [&](const char* vt, int kk, int cp) -> f16x8 {
    const int t = 16 * kk + t_lane;  // kk = 2 * token half + k-step
    const int j = 4 * cp + jl;
    const char* a0 = vt + t * kKRow + swz_v(t, j) + (ii & 1) * 8;
    const char* a1 = vt + (t + 8) * kKRow + swz_v(t + 8, j) + (ii & 1) * 8;
    return cat8(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)a0),
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)a1));
  };

  f32x16 O[4];
#pragma unroll
  for (int cp = 0; cp < 4; ++cp) O[cp] = f32x16{};
  float m_ref = -INFINITY;  // reference max of this lane's query (log2 units)
  float l_run = 0.f;        // this lane's share of sum 2^(x - m_ref)

  if (n_tiles > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int it = 0; it < n_tiles; ++it) {
    if (it + 1 < n_tiles) load(it + 1);
    const char* st = lds + (it & 1) * kMhaStage;
    const char* kt = st;
    const char* vt = st + kMhaTok * kKRow;
    const char* rt = st + 2 * kMhaTok * kKRow;

    // QK for both token halves
    f32x16 S[2];
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
      const int row = 32 * sh + lo;
      S[sh] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + row * kKRow + swz_k(row, 2 * ks + g));
        S[sh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], S[sh], 0, 0, 0);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(rt + row * kRRow + swz_r(row, 2 * ks + g));
        S[sh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[8 + ks], S[sh], 0, 0, 0);
      }
    }

    // scores in log2 units; the causal limit (and the sequence end) only
    // cut tiles past the block's first query's limit
    const int t0 = it * kMhaTok;
    float xs[2][16];
    const bool cut = t0 + kMhaTok > n_first;
#pragma unroll
    for (int sh = 0; sh < 2; ++sh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float v = S[sh][r] * scale_log2;
        const int t = t0 + 32 * sh + 8 * (r >> 2) + 4 * g + (r & 3);
        xs[sh][r] = (!cut || t < n_vis) ? v : -INFINITY;
      }
    float mt = -INFINITY;
#pragma unroll
    for (int sh = 0; sh < 2; ++sh)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, xs[sh][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    // raise the reference (and rescale what has been accumulated) only when
    // this tile's max exceeds it by more than the slack
    const bool raise = mt > m_ref + kRescaleSlack;
    if (__any(raise)) {
      const float nr = raise ? mt : m_ref;
      const float alpha = (raise && m_ref != -INFINITY) ? __builtin_amdgcn_exp2f(m_ref - nr) : (raise ? 0.f : 1.f);
#pragma unroll
      for (int cp = 0; cp < 4; ++cp)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[cp][r] *= alpha;
      l_run *= alpha;
      m_ref = nr;
    }
    f16x8 pb[4];
    const bool any_key = m_ref != -INFINITY;
#pragma unroll
    for (int sh = 0; sh < 2; ++sh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = any_key ? __builtin_amdgcn_exp2f(xs[sh][r] - m_ref) : 0.f;
        l_run += p;
        pb[2 * sh + (r >> 3)][r & 7] = (_Float16)p;
      }

    // PV over the tile's 4 k-steps of 16 tokens (P^T from this lane's scores)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int cp = 0; cp < 4; ++cp)
        O[cp] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vfrag(vt, kk, cp), pb[kk], O[cp], 0, 0, 0);

    if (it + 1 < n_tiles) store(it + 1);
    __syncthreads();
  }

  // ---- epilogue: lane owns query iq, dims 32cp + 8q + 4g + 0..3
  if (!q_live) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const int64_t row = ((int64_t)b * s_q + iq) * kH + h;
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  __bf16* orow = out + row * kDhc;
#pragma unroll
  for (int cp = 0; cp < 4; ++cp)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x4 o = {(__bf16)(O[cp][4 * q] * inv), (__bf16)(O[cp][4 * q + 1] * inv),
                        (__bf16)(O[cp][4 * q + 2] * inv), (__bf16)(O[cp][4 * q + 3] * inv)};
      *reinterpret_cast<bf16x4*>(orow + 32 * cp + 8 * q + 4 * g) = o;
    }
  if (g == 0) lse[row] = empty ? -INFINITY : (m_ref + __log2f(l_tot)) * 0.69314718055994531f;
}

hipError_t launch_prefill_mha(const __bf16* q_c, const __bf16* q_r, const __bf16* k_nope, const _Float16* v, int max_len,
                              const char* kv, int64_t num_pages, const int32_t* block_table, int max_pages,
                              const int32_t* seqlens, int B, int s_q, float scale_log2, __bf16* out, float* lse,
                              hipStream_t stream) {
  const int n_qb = (s_q + kMhaQ - 1) / kMhaQ;
  const int total = B * kH * n_qb;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL(prefill_mha_kernel, dim3(per_xcd * 8), dim3(256), 0, stream, q_c, q_r, k_nope, v, max_len, kv,
                     num_pages, block_table, max_pages, seqlens, s_q, scale_log2, out, lse, n_qb, B, total, per_xcd);
  return hipGetLastError();
}

}  // namespace mla
