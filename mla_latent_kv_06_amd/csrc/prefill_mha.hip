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
// filled with 16-byte direct-to-LDS loads: tile it+1 is requested right after
// the barrier that starts tile it, into the stage tile it-1 has released. One
// tile of lookahead is shorter than a memory round trip; the second
// workgroup on the CU (80 KiB of LDS each) computes while this one waits:
//   * QK: S^T[32 tokens, 32 queries] per token half on v_mfma_f32_32x32x16_bf16,
//     A = key rows from LDS, B = the wave's queries held in 48 VGPRs; a lane
//     owns one query and 16 of each 32 tokens;
//   * softmax in the exp2 domain against a per-query reference max taken from
//     the query's first tile; P = 2^(x - ref) may grow to 2^14 above it, which
//     fp16 P and the fp32 sums hold, so the accumulator is never rescaled (and
//     never touched by VALU). If a score exceeds its reference by more than
//     that, the workgroup rescans the block once with the exact maximum;
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
constexpr int kMhaStages = 2;
constexpr float kRefSlack = 14.f;                         // log2 units: P <= 2^14 < 65504 (fp16)

// 16-byte chunk positions: key rows (QK reads 16 consecutive rows at one
// chunk), value rows (transposed reads of 4 rows x 4 chunks), RoPE rows
__device__ __forceinline__ int swz_k(int row, int chunk) { return (chunk ^ (row & 15)) << 4; }
__device__ __forceinline__ int swz_v(int row, int chunk) { return (chunk ^ ((row & 3) << 2)) << 4; }
__device__ __forceinline__ int swz_r(int row, int chunk) { return (chunk ^ ((row >> 1) & 7)) << 4; }

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

// Workgroup barrier after this wave's own loads of the tile have been waited
// for with vmcnt; unlike __syncthreads() it does not drain the loads of the
// tiles still in flight.
__device__ __forceinline__ void tile_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Score accumulation kept in VGPRs (the softmax reads it with VALU) while
// the accumulator registers hold O^T. Written as asm: the first MFMA of a
// chain takes the literal 0 as its accumulator input (no zeroing moves), and
// a chain whose srcC is exactly the previous destination needs no wait
// states. The compiler cannot see the hazards of asm MFMAs: a VALU read of
// a v_mfma_f32_32x32x16_bf16 result needs 12 wait states on gfx950 (what the
// compiler's own hazard model inserts after the builtin), hence the fence tied
// to the value. It is 24 here, twice per tile: with two workgroups per CU the
// nops hand issue slots to the other workgroup's waves, and the minimal single
// fence measured 2 % slower (bit-identical results).
__device__ __forceinline__ void mfma_s_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_result_fence(f32x16& d) { asm("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(d)); }

__device__ __forceinline__ f16x8 cat8(i16x4 a, i16x4 b) {
  const f16x4 x = __builtin_bit_cast(f16x4, a), y = __builtin_bit_cast(f16x4, b);
  return f16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

}  // namespace

__global__ __launch_bounds__(256, 2) void prefill_mha_kernel(const __bf16* __restrict__ q_c, const __bf16* __restrict__ q_r,
                                                          const __bf16* __restrict__ k_nope,
                                                          const _Float16* __restrict__ v_in, int max_len,
                                                          const char* __restrict__ kv, int64_t num_pages,
                                                          const int32_t* __restrict__ block_table, int max_pages,
                                                          const int32_t* __restrict__ seqlens, int s_q, float scale_log2,
                                                          __bf16* __restrict__ out, float* __restrict__ lse,
                                                          int n_qb, int B, int total, int per_xcd) {
  __shared__ __attribute__((aligned(1024))) char lds[kMhaStages * kMhaStage];
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

  // ---- loader: wave w fills 1 KiB blocks 4w..4w+3 of the K and V regions
  // (rows 16w..16w+15) and blocks 2w, 2w+1 of the k_R region (rows
  // 16w..16w+15); lane l's slot in a block holds the logical chunk that the
  // swizzle puts there. Rows past L_b come from the zero-filled tail of the
  // last page of K and V (stage 1 writes it) and from the cache for k_R
  // (masked out of the scores).
  const char* kbase = reinterpret_cast<const char*>(k_nope + ((int64_t)b * kH + h) * max_len * kDhc);
  const char* vbase = reinterpret_cast<const char*>(v_in + ((int64_t)b * kH + h) * max_len * kDhc);
  unsigned koff[4], voff[4], roff[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * wave + 4 * j + (lane >> 4), ph = lane & 15;
    koff[j] = row * kKRow + ((ph ^ (row & 15)) << 4);
    voff[j] = row * kKRow + ((ph ^ ((row & 3) << 2)) << 4);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 16 * wave + 8 * j + (lane >> 3), ph = lane & 7;
    roff[j] = row * kRowBytes + kDc * 2 + ((ph ^ ((row >> 1) & 7)) << 4);
  }
  const unsigned lds0 = (unsigned)(uintptr_t)(lds_void_t*)lds;
  auto issue = [&](int it) {
    const unsigned st = lds0 + ((unsigned)it % (unsigned)kMhaStages) * kMhaStage;
    const char* ks = kbase + (int64_t)it * kMhaTok * kKRow;
    const char* vs = vbase + (int64_t)it * kMhaTok * kKRow;
    const char* rs = kv + physical_page(block_table, max_pages, b, it, num_pages) * kPageBytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dma16(ks, koff[j], st + (4 * wave + j) * 1024);
      dma16(vs, voff[j], st + kMhaTok * kKRow + (4 * wave + j) * 1024);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(rs, roff[j], st + 2 * kMhaTok * kKRow + (2 * wave + j) * 1024);
  };

  // ---- LDS read offsets, all lane constants plus compile-time immediates:
  // QK A operand: key row 32sh + lo, chunk 2ks + g (K: 8 k-steps, k_R: 4);
  // the row's swizzle depends only on lo. V^T operand: group G = lane >> 4,
  // ii = lane & 15 reads token row 4(G >> 1) + (ii >> 2) (+8 for the second
  // half, +16 per k-step, +32 per token half) and 4 columns 16(G & 1) +
  // 4(ii & 3) of a 32-column tile cp.
  int qk_k[8], qk_r[4], pv_v[4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qk_k[ks] = lo * kKRow + swz_k(lo, 2 * ks + g);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qk_r[ks] = 2 * kMhaTok * kKRow + lo * kRRow + swz_r(lo, 2 * ks + g);
  const int Gq = lane >> 4, ii = lane & 15;
  const int t_lane = 4 * (Gq >> 1) + (ii >> 2);
  const int jl = 2 * (Gq & 1) + ((ii & 3) >> 1);
#pragma unroll
  for (int cp = 0; cp < 4; ++cp)
    pv_v[cp] = kMhaTok * kKRow + t_lane * kKRow + swz_v(t_lane, 4 * cp + jl) + (ii & 1) * 8;

  f32x16 O[4];
  float m_ref = -INFINITY;   // reference max of this lane's query (log2 units)
  float m_seen = -INFINITY;  // true running max of this lane's query
  float l_run = 0.f;         // this lane's share of sum 2^(x - m_ref)

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int cp = 0; cp < 4; ++cp) O[cp] = f32x16{};
    l_run = 0.f;
    bool over = false;
    if (n_tiles > 0) issue(0);
    for (int it = 0; it < n_tiles; ++it) {
      // tile it has landed; after the barrier every wave is done with tile
      // it-1, whose stage is refilled with tile it+1 now
      wait_vmcnt<0>();
      tile_barrier();
      if (it + 1 < n_tiles) issue(it + 1);
      const char* st = lds + ((unsigned)it % (unsigned)kMhaStages) * kMhaStage;  // unsigned: lets the reads fold immediates

      // QK for both token halves (raw scores; the scale is applied in the exp),
      // in program order: the key fragment of MFMA k+3 is read right after
      // MFMA k, so three LDS reads are in flight and no more registers are held
      f32x16 S[2];
      {
        auto kfrag = [&](int k) -> bf16x8 {  // k = 12 sh + ks
          const int sh = k / 12, ks = k % 12;
          const int off = ks < 8 ? qk_k[ks] + sh * 32 * kKRow : qk_r[ks - 8] + sh * 32 * kRRow;
          return *reinterpret_cast<const bf16x8*>(st + off);
        };
        bf16x8 kf[4];
#pragma unroll
        for (int k = 0; k < 3; ++k) kf[k] = kfrag(k);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < 24; ++k) {
          const int sh = k / 12, ks = k % 12;
          if (ks == 0)
            mfma_s_first(S[sh], kf[k & 3], qf[ks]);
          else
            mfma_s(S[sh], kf[k & 3], qf[ks]);
          if (k + 3 < 24) kf[(k + 3) & 3] = kfrag(k + 3);
          __builtin_amdgcn_sched_barrier(0);
        }
        mfma_result_fence(S[0]);
        mfma_result_fence(S[1]);
        __builtin_amdgcn_sched_barrier(0);
      }

      // the causal limit (and the sequence end) only cut tiles past the
      // block's first query's limit: one uniform branch, taken rarely
      const int t0 = it * kMhaTok;
      if (t0 + kMhaTok > n_first) {
        const int lim = n_vis - t0 - 4 * g;  // token t0 + 32sh + 8(r>>2) + 4g + (r&3) is visible iff below n_vis
#pragma unroll
        for (int sh = 0; sh < 2; ++sh)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            S[sh][r] = (32 * sh + 8 * (r >> 2) + (r & 3)) < lim ? S[sh][r] : -INFINITY;
      }
      // softmax_scale > 0, so the max of the raw scores gives the max of the
      // scaled ones
      float mt = fmaxf(S[0][0], S[0][1]);
#pragma unroll
      for (int r = 2; r < 16; ++r) mt = fmaxf(mt, S[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, S[1][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * scale_log2;
      // the first tile with a visible key sets the reference (nothing has been
      // accumulated yet); later tiles only record whether they outgrew it
      m_seen = fmaxf(m_seen, mt);
      if (m_ref == -INFINITY) m_ref = mt;
      over |= mt > m_ref + kRefSlack;
      // P = 2^(s * scale_log2 - m_ref) in one fma; masked scores give 0, and
      // while this lane's query has seen no key all its scores are masked (an
      // offset of 0 keeps -inf - (-inf) out)
      const float off = m_ref == -INFINITY ? 0.f : -m_ref;
      f16x8 pb[4];
#pragma unroll
      for (int sh = 0; sh < 2; ++sh)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[sh][r], scale_log2, off));
          l_run += p;
          pb[2 * sh + (r >> 3)][r & 7] = (_Float16)p;
        }

      // PV over the tile's 4 k-steps of 16 tokens (P^T from this lane's
      // scores); V^T fragments through four per-tile bases plus immediates,
      // read two MFMAs ahead
      {
        const char* vb[4];
#pragma unroll
        for (int cp = 0; cp < 4; ++cp) vb[cp] = st + pv_v[cp];
        auto vfrag = [&](int k) -> f16x8 {  // k = 4 kk + cp
          const char* a = vb[k & 3] + (k >> 2) * 16 * kKRow;
          return cat8(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)a),
                      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a + 8 * kKRow)));
        };
        f16x8 vf[3];
        vf[0] = vfrag(0);
        vf[1] = vfrag(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          O[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[k % 3], pb[k >> 2], O[k & 3], 0, 0, 0);
          if (k + 2 < 16) vf[(k + 2) % 3] = vfrag(k + 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // every score within the slack of its reference: done; otherwise rescan
    // the block once with the exact maxima (which cannot be exceeded). The
    // per-wave flags go through the (now idle) start of the LDS ring.
    __syncthreads();
    int* flags = reinterpret_cast<int*>(lds);
    const bool wave_over = __any(over);
    if (lane == 0) flags[wave] = wave_over ? 1 : 0;
    __syncthreads();
    const bool again = (flags[0] | flags[1] | flags[2] | flags[3]) != 0;
    if (!again || pass == 1) break;
    __syncthreads();  // every wave has read the flags before the rescan's loads land
    m_ref = m_seen;
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
