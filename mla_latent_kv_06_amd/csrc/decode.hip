// Stage 1 of absorbed MLA decode: split scan of the paged latent cache.
//
// One workgroup = one (sequence b, query i, split s) work item and all 128
// heads, so every 1152-byte cache row is fetched from HBM once per work item
// and shared by all heads through LDS (absorbed scores of the MLA
// operator-teardown page, section 4; split scan of the K3 time-share study,
// "Inside the blocks").
//
// Layout of the work:
//   * 4 waves; wave w owns heads 32w..32w+31.
//   * the cache streams through a ring of 4 LDS stages of 32 tokens (36 KiB
//     each, half a page); three stages are in flight while one is consumed.
//     Stages are filled with 16-byte direct-to-LDS loads, 9 per thread.
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: A = 32 cache rows x 16 dims
//     read from LDS, B = the wave's 32 queries (held in 144 VGPRs for all
//     576 dims). Each lane ends up owning one head and 16 of the tile's
//     tokens; its partner lane (lane ^ 32) owns the other 16.
//   * softmax in the exp2 domain against a per-head reference max taken from
//     the split's first tile; P = exp2(x - ref) may grow to 2^64, which bf16
//     and the fp32 accumulators hold without loss, so the accumulator is
//     never rescaled. Each lane also tracks the true running max; if any
//     score exceeded its reference by more than 64, the workgroup rescans
//     the split once with the exact max as reference (only adversarial
//     score ranges trigger it; a second rescan is impossible).
//   * O^T += V^T . P^T on the same MFMA: the S accumulator registers are
//     already the P^T operand layout, and V^T is read from the row-major
//     tile with ds_read_b64_tr_b16 (each 16-lane group turns a 4-row x
//     16-column block into 4 consecutive tokens per lane). O^T (512 x 32
//     per wave) lives in the accumulation registers.
//   * LDS rows are 72 chunks of 16 bytes; the low 3 bits of a chunk index are
//     XOR-swizzled with ((t&3)<<1) ^ ((t>>2)&7) of the row t, which keeps both
//     the 16-byte row reads of QK and the transposed 8-byte reads of PV free
//     of bank conflicts.
#include "mla_device.hpp"
#include "decode.hpp"

namespace mla {

namespace {

constexpr int kTok = 32;                          // tokens per LDS stage
constexpr int kStages = 4;                        // LDS ring depth
constexpr int kStageBytes = kTok * kRowBytes;     // 36864
constexpr int kThreads = 256;
constexpr int kDmaPerThread = kStageBytes / (kThreads * 16);  // 9
constexpr float kRefSlack = 64.0f;                // log2 headroom above the reference max
static_assert(kDmaPerThread * kThreads * 16 == kStageBytes, "stage must split into 16-byte loads");

__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) ^ ((t >> 2) & 7); }

__device__ __forceinline__ float shfl_xor32(float v) { return __shfl_xor(v, 32, 64); }

// S^T accumulation kept in VGPRs (the softmax reads it with VALU) while the
// 256 AGPRs hold O^T. Only this MFMA is written as asm: a chain whose srcC is
// exactly the previous destination needs no wait states.
__device__ __forceinline__ void mfma_qk_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_qk(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// VALU may read an MFMA result only after the MFMA has drained (at most
// 16 passes + 2 on CDNA; 24 wait states here). Tied to the value so no read
// of it can be scheduled above the wait.
__device__ __forceinline__ void mfma_result_fence(f32x16& d) {
  asm("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(d));
}

}  // namespace

__global__ __launch_bounds__(kThreads) void decode_paged_kernel(
    const __bf16* __restrict__ q_abs, const __bf16* __restrict__ q_r, const char* __restrict__ kv,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seqlens,
    float* __restrict__ o_part, float* __restrict__ lse_part, DecodeParams a) {
  __shared__ __attribute__((aligned(1024))) char lds[kStages * kStageBytes];
  __shared__ int rescan_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lo = lane & 31;
  const int g = lane >> 5;

  // blockIdx -> work item, contiguous per XCD (workgroups are dealt to the 8
  // XCDs round-robin), so neighbouring items share an L2.
  const int x = blockIdx.x;
  const int item = (x & 7) * a.items_per_xcd + (x >> 3);
  if (item >= a.items) return;
  const int i = item % a.s_q;
  const int rest = item / a.s_q;
  const int split = rest % a.num_splits;
  const int b = rest / a.num_splits;

  const int L = clamp_len(seqlens[b], a.max_pages);
  int Lv = L - a.s_q + i + 1;  // keys visible to query i
  if (Lv < 0) Lv = 0;
  const int n_pages = (Lv + kPage - 1) / kPage;
  const int per = (n_pages + a.num_splits - 1) / a.num_splits;
  const int p0 = min(split * per, n_pages);
  const int p1 = min(p0 + per, n_pages);
  const int t_begin = p0 * kPage;
  const int t_end = min(p1 * kPage, Lv);
  const int tile0 = t_begin / kTok;
  const int n_tiles = t_end > t_begin ? (t_end - t_begin + kTok - 1) / kTok : 0;

  const int h = wave * 32 + lo;
  const int64_t qrow = (int64_t)(b * a.s_q + i) * kH + h;
  const int64_t orow = qrow * a.num_splits + split;

  if (tid == 0) rescan_flag = 0;

  // queries: B operand of S^T = K . Q^T; lane (g, lo) holds dims 16kk+8g..+7 of head h
  bf16x8 qf[36];
  if (n_tiles > 0) {
    const bf16x8* qa = reinterpret_cast<const bf16x8*>(q_abs + qrow * kDc);
    const bf16x8* qr = reinterpret_cast<const bf16x8*>(q_r + qrow * kDr);
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) qf[kk] = qa[2 * kk + g];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[32 + kk] = qr[2 * kk + g];
  }

  // QK A operand: row lo, chunk 2kk+g; kk = 4a + r -> offset qk_off[r] + 128a
  int qk_off[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) qk_off[r] = lo * kRowBytes + (((2 * r + g) ^ swz(lo)) << 4);
  // PV A operand (V^T) through transposed reads; group G = lane>>4, ii = lane&15
  // fetches row 4(G>>1) + (ii>>2) (+8 half, +16 ks), columns 16(G&1) + 4(ii&3)..+3
  int pv_off[2][2][2];  // [ct&1][half][ks]
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
          pv_off[cp][hf][ks] = t * kRowBytes + ((j ^ swz(t)) << 4) + (ii & 1) * 8;
        }
  }

  // DMA: thread tid fills chunk slot q = k*256 + tid of a stage; the matching
  // source chunk of the 32-row half page is (row q/72, chunk (q%72) ^ swz(row))
  unsigned dma_off[kDmaPerThread];
#pragma unroll
  for (int k = 0; k < kDmaPerThread; ++k) {
    const unsigned q = k * kThreads + tid;
    const unsigned t = q / 72u;
    const unsigned p = q - t * 72u;
    dma_off[k] = t * kRowBytes + ((p ^ swz(t)) << 4);
  }
  auto issue = [&](int tile, int stage) {
    const int64_t page = physical_page(block_table, a.max_pages, b, tile >> 1, a.num_pages);
    const char* src = kv + page * kPageBytes + (tile & 1) * kStageBytes;
    char* dst = lds + stage * kStageBytes + wave * 1024;
#pragma unroll
    for (int k = 0; k < kDmaPerThread; ++k) {
      // keep the 32-bit offset opaque inside the loop so that the address is
      // formed as uniform base + 32-bit lane offset (no 64-bit copies hoisted)
      unsigned off = dma_off[k];
      asm volatile("" : "+v"(off));
      __builtin_amdgcn_global_load_lds(src + off, (lds_void_t*)(dst + k * (kThreads * 16)), 16, 0, 0);
    }
  };

  const float c_log2 = a.scale_log2;
  f32x16 O[16];
  float m_ref = -INFINITY;   // reference max of this head (log2 units)
  float m_seen = -INFINITY;  // true running max of this head
  float l_run = 0.f;         // this lane's share of sum exp2(x - m_ref)

  for (int pass = 0; pass < 2; ++pass) {
    // O^T = 0 through the matrix core, so O is only ever defined by MFMAs
    {
      const bf16x8 z = bf16x8{};
#pragma unroll
      for (int ct = 0; ct < 16; ++ct) O[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(z, z, f32x16{}, 0, 0, 0);
    }
    l_run = 0.f;
    bool over = false;

    const int pre = n_tiles < kStages - 1 ? n_tiles : kStages - 1;
    for (int s = 0; s < pre; ++s) issue(tile0 + s, s);

    for (int it = 0; it < n_tiles; ++it) {
      const int ahead = n_tiles - 1 - it;
      if (ahead >= 2)
        wait_vmcnt<2 * kDmaPerThread>();
      else if (ahead == 1)
        wait_vmcnt<kDmaPerThread>();
      else
        wait_vmcnt<0>();
      __syncthreads();
      if (it + kStages - 1 < n_tiles) issue(tile0 + it + kStages - 1, (it + kStages - 1) & (kStages - 1));

      char* tb = lds + (it & (kStages - 1)) * kStageBytes;
      const int valid = t_end - (tile0 + it) * kTok;  // >= 1; >= 32 means a full tile
      if (valid < kTok) {
        // rows past the visible length may hold anything (even NaN); P is 0
        // there, so make those rows exactly 0 as well
        for (int q = tid; q < (kTok - valid) * (kRowBytes / 16); q += kThreads)
          *reinterpret_cast<f32x4*>(tb + valid * kRowBytes + q * 16) = f32x4{};
        __syncthreads();
      }

      // ---- S^T[token, head] over 576 dims
      f32x16 S;
      mfma_qk_first(S, *reinterpret_cast<const bf16x8*>(tb + qk_off[0]), qf[0]);
#pragma unroll
      for (int kk = 1; kk < 36; ++kk)
        mfma_qk(S, *reinterpret_cast<const bf16x8*>(tb + qk_off[kk & 3] + (kk >> 2) * 128), qf[kk]);
      mfma_result_fence(S);

      // ---- softmax numerators (lane owns head h, tokens 8(r>>2) + 4g + (r&3))
      float xs[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) xs[r] = S[r] * c_log2;
      if (valid < kTok) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = 8 * (r >> 2) + 4 * g + (r & 3);
          if (tok >= valid) xs[r] = -INFINITY;
        }
      }
      float mx = xs[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, xs[r]);
      mx = fmaxf(mx, shfl_xor32(mx));
      m_seen = fmaxf(m_seen, mx);
      if (m_ref == -INFINITY) m_ref = mx;  // first tile of the first pass
      over |= mx > m_ref + kRefSlack;
      bf16x8 pb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(xs[r] - m_ref);
        l_run += p;
        pb[r >> 3][r & 7] = (__bf16)p;
      }

      // ---- O^T[c, head] += V^T[c, token] . P^T[token, head]
      // 32 MFMAs n = 2ct + ks; the V^T fragments are read 3 MFMAs ahead
      auto vfrag = [&](int n) {
        const int ct = n >> 1, ks = n & 1;
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(tb + pv_off[ct & 1][0][ks] + (ct >> 1) * 128));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(tb + pv_off[ct & 1][1][ks] + (ct >> 1) * 128));
        const bf16x4 b0 = __builtin_bit_cast(bf16x4, v0);
        const bf16x4 b1 = __builtin_bit_cast(bf16x4, v1);
        return bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      };
      bf16x8 vq[4];
      vq[0] = vfrag(0);
      vq[1] = vfrag(1);
      vq[2] = vfrag(2);
#pragma unroll
      for (int n = 0; n < 32; ++n) {
        if (n + 3 < 32) vq[(n + 3) & 3] = vfrag(n + 3);
        O[n >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vq[n & 3], pb[n & 1], O[n >> 1], 0, 0, 0);
      }
      // schedule: the first three fragments (6 reads), then per MFMA the reads
      // of the fragment three MFMAs ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int n = 0; n < 29; ++n) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    }

    // rescan once with the exact max if some score outgrew its reference
    if (__any(over) && lane == 0) rescan_flag = 1;
    __syncthreads();
    const bool again = rescan_flag != 0;
    if (!again || pass == 1) break;
    __syncthreads();
    m_ref = m_seen;
  }

  // ---- epilogue: normalise, write this split's partial row and its LSE
  const float l_tot = l_run + shfl_xor32(l_run);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.0f / l_tot;
  float* orow_ptr = o_part + orow * kDc;
#pragma unroll
  for (int ct = 0; ct < 16; ++ct)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = empty ? 0.f : O[ct][4 * q + e] * inv;
      *reinterpret_cast<f32x4*>(orow_ptr + 32 * ct + 8 * q + 4 * g) = v;
    }
  if (g == 0)
    lse_part[orow] = empty ? -INFINITY : (m_ref + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f;
}

hipError_t launch_decode_paged(const DecodeParams& p, hipStream_t stream) {
  const int blocks = 8 * p.items_per_xcd;
  hipLaunchKernelGGL(decode_paged_kernel, dim3(blocks), dim3(kThreads), 0, stream, p.q_abs, p.q_r, p.kv,
                     p.block_table, p.seqlens, p.o_part, p.lse_part, p);
  return hipGetLastError();
}

}  // namespace mla
