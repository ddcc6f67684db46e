// mla_decode_step_static: the decode step with no caller workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation). The absorbed
// queries and the split partials, which mla_decode_step takes as
// caller-owned buffers, live here in one file-scope device array.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>

#include "../../include/mla.h"
#include "decode.hpp"
#include "validate.hpp"

namespace {

// One copy per GPU, loaded with the module and held until the process ends.
// Host code never takes its address directly: the name stands for a
// host-side shadow, so device addresses come from hipGetSymbolAddress.
__device__ __align__(256) char scratch[mla::kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
hipError_t scratch_on_current_device(void** ptr, int* dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  *dev_out = dev;
  return hipSuccess;
}

}  // namespace

// status detail shared with mla_last_error (defined in mla_api.hip)
void mla_set_last_error(const std::string& s);

extern "C" mla_status mla_decode_step_static(const void* q_c, const void* q_r, const void* kv_cache,
                                             int64_t num_pages, const int32_t* block_table, int max_pages,
                                             const int32_t* seqlens, int B, int s_q, int H, const void* w_uk,
                                             const void* w_uv, float softmax_scale, int num_splits, void* out,
                                             float* lse, void* stream) {
  const mla::Check c = mla::check_step_static(q_c, q_r, kv_cache, num_pages, block_table, max_pages, seqlens, B, s_q,
                                              H, w_uk, w_uv, softmax_scale, num_splits, out, lse);
  if (!c.ok()) {
    mla_set_last_error(c.detail);
    return c.status;
  }
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  void* base = nullptr;
  int dev = -1;
  hipError_t e = scratch_on_current_device(&base, &dev);
  if (e == hipSuccess && st != nullptr) {
    int sdev = -1;
    e = hipStreamGetDevice(st, &sdev);
    if (e == hipSuccess && sdev != dev) {
      mla_set_last_error("mla_decode_step_static: the stream belongs to device " + std::to_string(sdev) +
                         " but device " + std::to_string(dev) + " is current");
      return MLA_ERR_HIP;
    }
  }
  if (e != hipSuccess) {
    mla_set_last_error(std::string("mla_decode_step_static scratch lookup: ") + hipGetErrorString(e));
    return MLA_ERR_HIP;
  }
  const mla::ScratchLayout L = mla::scratch_layout(B, s_q, num_splits);
  char* const sp = static_cast<char*>(base);
  __bf16* const q_abs = reinterpret_cast<__bf16*>(sp + L.q_abs);
  float* const o_part = reinterpret_cast<float*>(sp + L.o_part);
  float* const lse_part = reinterpret_cast<float*>(sp + L.lse_part);
  const int T = B * s_q;
  // every partial slot the merge reads is written by the scan (empty slots get
  // LSE -inf and are never read), so nothing in the array has to be cleared
  e = mla::launch_absorb(static_cast<const __bf16*>(q_c), static_cast<const __bf16*>(w_uk), q_abs, T, st);
  if (e == hipSuccess) {
    mla::DecodeParams p{};
    p.q_abs = q_abs;
    p.q_r = static_cast<const __bf16*>(q_r);
    p.kv = static_cast<const char*>(kv_cache);
    p.num_pages = num_pages;
    p.block_table = block_table;
    p.max_pages = max_pages;
    p.seqlens = seqlens;
    p.B = B;
    p.s_q = s_q;
    p.num_splits = num_splits;
    p.scale_log2 = softmax_scale * 1.44269504088896340736f;
    p.o_part = o_part;
    p.lse_part = lse_part;
    e = mla::launch_decode_paged(p, st);
  }
  if (e == hipSuccess)
    e = mla::launch_combine_up(o_part, lse_part, static_cast<const __bf16*>(w_uv), T, num_splits,
                               static_cast<__bf16*>(out), lse, st);
  if (e != hipSuccess) {
    mla_set_last_error(std::string("mla_decode_step_static launch: ") + hipGetErrorString(e));
    return MLA_ERR_HIP;
  }
  return MLA_OK;
}
