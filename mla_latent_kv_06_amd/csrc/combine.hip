// Stage 2 kernel (body in combine_body.hpp).
#include "combine_body.hpp"

namespace mla {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part, int rows,
                                                      int num_splits, float* __restrict__ o_lat,
                                                      float* __restrict__ lse) {
  combine_body(blockIdx.x, o_part, lse_part, rows, num_splits, o_lat, lse);
}

hipError_t launch_combine(const float* o_part, const float* lse_part, int rows, int num_splits,
                          float* o_lat, float* lse, hipStream_t stream) {
  const int blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, stream, o_part, lse_part, rows, num_splits,
                     o_lat, lse);
  return hipGetLastError();
}

}  // namespace mla
