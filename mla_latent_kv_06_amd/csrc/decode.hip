// Stage 1 of absorbed MLA decode as a kernel of its own: the split scan of
// decode_body.hpp, one workgroup per MI355X CU.
#include "decode_body.hpp"

namespace mla {

template <bool kStream, int kFmt>
__global__ __launch_bounds__(kDecodeThreads) void decode_paged_kernel(
    const __bf16* __restrict__ q_abs, const __bf16* __restrict__ q_r, const char* __restrict__ kv,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seqlens,
    float* __restrict__ o_part, float* __restrict__ lse_part, DecodeParams a) {
  __shared__ __attribute__((aligned(1024))) char lds[decode_lds_bytes<kFmt>()];
  decode_paged_body<kStream, kFmt>(lds, q_abs, q_r, kv, block_table, seqlens, o_part, lse_part, a);
}

hipError_t launch_decode_paged(const DecodeParams& p, hipStream_t stream) {
  if (p.s_q == 1)
    hipLaunchKernelGGL((decode_paged_kernel<true, kFmtBf16>), dim3(kDecodeGroups), dim3(kDecodeThreads), 0, stream, p.q_abs,
                       p.q_r, p.kv, p.block_table, p.seqlens, p.o_part, p.lse_part, p);
  else
    hipLaunchKernelGGL((decode_paged_kernel<false, kFmtBf16>), dim3(kDecodeGroups), dim3(kDecodeThreads), 0, stream, p.q_abs,
                       p.q_r, p.kv, p.block_table, p.seqlens, p.o_part, p.lse_part, p);
  return hipGetLastError();
}

hipError_t launch_decode_paged_fp8(const DecodeParams& p, hipStream_t stream) {
  if (p.s_q == 1)
    hipLaunchKernelGGL((decode_paged_kernel<true, kFmtFp8>), dim3(kDecodeGroups), dim3(kDecodeThreads), 0, stream, p.q_abs,
                       p.q_r, p.kv, p.block_table, p.seqlens, p.o_part, p.lse_part, p);
  else
    hipLaunchKernelGGL((decode_paged_kernel<false, kFmtFp8>), dim3(kDecodeGroups), dim3(kDecodeThreads), 0, stream, p.q_abs,
                       p.q_r, p.kv, p.block_table, p.seqlens, p.o_part, p.lse_part, p);
  return hipGetLastError();
}

hipError_t launch_decode_paged_mxfp4(const DecodeParams& p, hipStream_t stream) {
  if (p.s_q == 1)
    hipLaunchKernelGGL((decode_paged_kernel<true, kFmtMxfp4>), dim3(kDecodeGroups), dim3(kDecodeThreads), 0, stream,
                       p.q_abs, p.q_r, p.kv, p.block_table, p.seqlens, p.o_part, p.lse_part, p);
  else
    hipLaunchKernelGGL((decode_paged_kernel<false, kFmtMxfp4>), dim3(kDecodeGroups), dim3(kDecodeThreads), 0, stream,
                       p.q_abs, p.q_r, p.kv, p.block_table, p.seqlens, p.o_part, p.lse_part, p);
  return hipGetLastError();
}

}  // namespace mla
