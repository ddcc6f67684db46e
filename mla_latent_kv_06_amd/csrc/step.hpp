// Launch interface of the one-launch decode step (step.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "decode.hpp"

namespace mla {

struct StepParams {
  DecodeParams d;           // the scan's arguments; d.q_abs is written by phase 1
  const __bf16* q_c;        // [B, s_q, 128, 128]
  const __bf16* w_uk;       // [128, 128, 512]
  const __bf16* w_uv;       // [128, 128, 512]
  float* o_lat;             // [B, s_q, 128, 512] (written by phase 3)
  float* lse;               // [B, s_q, 128]
  __bf16* out;              // [B, s_q, 128, 128]
};

// Cooperative launch of 256 workgroups (one per CU); fails with the runtime's
// error if they cannot all be resident.
hipError_t launch_decode_step(const StepParams& p, int fmt, hipStream_t stream);  // fmt: kFmt* of decode.hpp

}  // namespace mla
