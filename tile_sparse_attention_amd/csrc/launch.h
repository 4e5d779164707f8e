// Kernel launchers called by the C ABI layer (api.cpp).  Each returns the
// launch status; arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsa.h"

namespace tsa {

struct AttnLaunch {
  const tsa_problem_t* p;
  const void* q;
  const void* k;
  const void* v;
  const uint32_t* mask;
  float scale;
  void* o;
  float* lse;
  hipStream_t stream;
};

hipError_t launch_attention_bf16(const AttnLaunch& a);
hipError_t launch_attention_f32(const AttnLaunch& a);

}  // namespace tsa
