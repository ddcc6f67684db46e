// Kernels of the per-head projections (bodies in gemm_body.hpp).
#include "gemm_body.hpp"

namespace mla {

__global__ __launch_bounds__(256) void absorb_kernel(const __bf16* __restrict__ q_c, const __bf16* __restrict__ w_uk,
                                                     __bf16* __restrict__ q_abs, int T) {
  __shared__ __attribute__((aligned(16))) char lds[kAbsorbLdsBytes];
  // workgroup x: item x mod 512 (so all token blocks of an item run on one XCD
  // and share its W_UK block in L2), tokens of block x / 512
  const int t_begin = (blockIdx.x / kAbsorbItems) * kAbsorbTokens;
  absorb_body(lds, blockIdx.x % kAbsorbItems, q_c, w_uk, q_abs, t_begin, min(T, t_begin + kAbsorbTokens));
}

__global__ __launch_bounds__(256) void up_proj_kernel(const float* __restrict__ o_lat, const __bf16* __restrict__ w_uv,
                                                      __bf16* __restrict__ out, int T, int wg_per_xcd) {
  __shared__ f32x4 red[4][4][64];  // [wave][register quad][lane]
  up_proj_body(red, blockIdx.x, o_lat, w_uv, out, T, wg_per_xcd);
}

hipError_t launch_absorb(const __bf16* q_c, const __bf16* w_uk, __bf16* q_abs, int T, hipStream_t stream) {
  const int blocks = (T + kAbsorbTokens - 1) / kAbsorbTokens;
  hipLaunchKernelGGL(absorb_kernel, dim3(kAbsorbItems * blocks), dim3(256), 0, stream, q_c, w_uk, q_abs, T);
  return hipGetLastError();
}

hipError_t launch_up_proj(const float* o_lat, const __bf16* w_uv, __bf16* out, int T, hipStream_t stream) {
  constexpr int kWg = kUpProjItems;
  constexpr int kPerXcd = kWg / 8;
  hipLaunchKernelGGL(up_proj_kernel, dim3(kWg), dim3(256), 0, stream, o_lat, w_uv, out, T, kPerXcd);
  return hipGetLastError();
}

}  // namespace mla
