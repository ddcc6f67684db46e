// Debug/test aid: gather the logical cache rows of each sequence through the
// block table with the same page arithmetic (token_row) the decode uses, so
// tests can check the paged indexing byte for byte.
#include "mla_device.hpp"
#include "decode.hpp"

namespace mla {

__global__ __launch_bounds__(256) void gather_kernel(const char* __restrict__ kv, int64_t num_pages,
                                                     const int32_t* __restrict__ block_table, int max_pages,
                                                     const int32_t* __restrict__ seqlens, int B, int max_len,
                                                     __bf16* __restrict__ out) {
  constexpr int kChunks = kRowBytes / 16;  // 72 chunks of 16 bytes per row
  const int64_t total = (int64_t)B * max_len * kChunks;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += (int64_t)gridDim.x * blockDim.x) {
    const int ch = (int)(q % kChunks);
    const int64_t bt = q / kChunks;
    const int t = (int)(bt % max_len);
    const int b = (int)(bt / max_len);
    const int L = clamp_len(seqlens[b], max_pages);
    f32x4 v = f32x4{};
    if (t < L) v = *reinterpret_cast<const f32x4*>(token_row(kv, block_table, max_pages, b, t, num_pages) + ch * 16);
    *reinterpret_cast<f32x4*>(reinterpret_cast<char*>(out) + bt * kRowBytes + ch * 16) = v;
  }
}

hipError_t launch_gather(const char* kv, int64_t num_pages, const int32_t* block_table, int max_pages,
                         const int32_t* seqlens, int B, int max_len, __bf16* out, hipStream_t stream) {
  const int64_t total = (int64_t)B * max_len * (kRowBytes / 16);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, kv, num_pages, block_table, max_pages,
                     seqlens, B, max_len, out);
  return hipGetLastError();
}

}  // namespace mla
