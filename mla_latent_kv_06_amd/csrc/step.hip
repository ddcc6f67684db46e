// The whole absorbed decode step in one launch: absorb -> split scan ->
// split merge -> per-head up-projection, as phases of one persistent kernel
// separated by grid-wide barriers.
//
// At 4K context the K3 time-share study ("Inside the blocks") measures the
// split merge and the projections around the scan at several times the scan
// itself. Here the step is one launch, and each phase runs
// the workgroup body of the corresponding kernel (gemm_body.hpp,
// decode_body.hpp, combine_body.hpp) over a grid-stride loop of its work
// items, so the results are bit-identical to launching mla_absorb_q,
// mla_decode_paged, mla_combine_splits and mla_up_proj one after another.
//
// The grid is the scan's: 256 workgroups of 256 threads, one per MI355X CU
// (the scan's 160 KiB of LDS, reused by every phase, admits one per CU). The
// launch is cooperative, so the runtime either makes all 256 co-resident or
// refuses the launch; a barrier therefore cannot wait on a workgroup that
// never runs. Intermediates (q_abs, the split partials, o_lat) live in
// caller-owned buffers, as with the separate kernels.
#include <hip/hip_cooperative_groups.h>

#include "combine_body.hpp"
#include "decode_body.hpp"
#include "gemm_body.hpp"
#include "step.hpp"

namespace mla {

namespace {

template <int kFmt>
constexpr bool phases_fit() {
  return kAbsorbLdsBytes <= decode_lds_bytes<kFmt>() && kUpProjLdsBytes <= decode_lds_bytes<kFmt>();
}
static_assert(phases_fit<kFmtBf16>() && phases_fit<kFmtFp8>() && phases_fit<kFmtMxfp4>(),
              "every phase fits in the scan's LDS, for every cache format");

}  // namespace

// Every buffer is its own __restrict__ argument (not a struct field), so the
// compiler can prove that no store of an earlier phase touches the block table
// or the lengths and keeps their uniform loads on the scalar path, as in the
// scan kernel; q_abs and o_lat are written by one phase and read by a later
// one through the same pointer, after a grid barrier.
template <bool kStream, int kFmt>
__global__ __launch_bounds__(kDecodeThreads) void decode_step_kernel(
    const __bf16* __restrict__ q_c, const __bf16* __restrict__ w_uk, const __bf16* __restrict__ w_uv,
    __bf16* __restrict__ q_abs, const __bf16* __restrict__ q_r, const char* __restrict__ kv,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seqlens, float* __restrict__ o_part,
    float* __restrict__ lse_part, float* __restrict__ o_lat, float* __restrict__ lse, __bf16* __restrict__ out,
    DecodeParams a) {
  __shared__ __attribute__((aligned(1024))) char lds[decode_lds_bytes<kFmt>()];
  cooperative_groups::grid_group grid = cooperative_groups::this_grid();
  const int T = a.B * a.s_q;

  // phase 1: q_abs = q_c . W_UK, work items (head, 128-column block)
  for (int item = blockIdx.x; item < kAbsorbItems; item += gridDim.x) {
    absorb_body(lds, item, q_c, w_uk, q_abs, 0, T);
    __syncthreads();  // the next item restages the weights in LDS
  }
  grid.sync();
  // nothing of phase 1 is in flight; saying so keeps the compiler from
  // guarding the scan's registers with waits that would also drain its
  // (untracked) tile loads
  wait_vmcnt<0>();

  // phase 2: the split scan, workgroup k scanning page range k
  decode_paged_body<kStream, kFmt>(lds, q_abs, q_r, kv, block_table, seqlens, o_part, lse_part, a);
  grid.sync();

  // phase 3: merge the partials of each (token, head) row, four rows per item
  const int rows = T * kH;
  for (int item = blockIdx.x; item < (rows + 3) / 4; item += gridDim.x)
    combine_body(item, o_part, lse_part, rows, a.num_splits, o_lat, lse);
  grid.sync();

  // phase 4: out = o_lat . W_UV^T per head; item x keeps its XCD (x & 7)
  for (int x = blockIdx.x; x < kUpProjItems; x += gridDim.x) {
    up_proj_body(reinterpret_cast<f32x4(*)[4][64]>(lds), x, o_lat, w_uv, out, T, kUpProjItems / 8);
    __syncthreads();  // the next item reuses the reduction buffer
  }
}

hipError_t launch_decode_step(const StepParams& p, int fmt, hipStream_t stream) {
  const void* fn;
  const bool stream1 = p.d.s_q == 1;
  if (fmt == kFmtFp8)
    fn = stream1 ? reinterpret_cast<const void*>(&decode_step_kernel<true, kFmtFp8>)
                 : reinterpret_cast<const void*>(&decode_step_kernel<false, kFmtFp8>);
  else if (fmt == kFmtMxfp4)
    fn = stream1 ? reinterpret_cast<const void*>(&decode_step_kernel<true, kFmtMxfp4>)
                 : reinterpret_cast<const void*>(&decode_step_kernel<false, kFmtMxfp4>);
  else
    fn = stream1 ? reinterpret_cast<const void*>(&decode_step_kernel<true, kFmtBf16>)
                 : reinterpret_cast<const void*>(&decode_step_kernel<false, kFmtBf16>);
  const __bf16* q_c = p.q_c;
  const __bf16* w_uk = p.w_uk;
  const __bf16* w_uv = p.w_uv;
  __bf16* q_abs = const_cast<__bf16*>(p.d.q_abs);
  const __bf16* q_r = p.d.q_r;
  const char* kv = p.d.kv;
  const int32_t* bt = p.d.block_table;
  const int32_t* sl = p.d.seqlens;
  float* o_part = p.d.o_part;
  float* lse_part = p.d.lse_part;
  float* o_lat = p.o_lat;
  float* lse = p.lse;
  __bf16* out = p.out;
  DecodeParams a = p.d;
  void* args[] = {&q_c, &w_uk, &w_uv, &q_abs, &q_r, &kv, &bt, &sl, &o_part, &lse_part, &o_lat, &lse, &out, &a};
  return hipLaunchCooperativeKernel(fn, dim3(kDecodeGroups), dim3(kDecodeThreads), args, 0, stream);
}

}  // namespace mla
