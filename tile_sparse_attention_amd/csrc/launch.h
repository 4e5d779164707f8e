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
  void* workspace;  // packed V^T, attention_vt_bytes() bytes
  hipStream_t stream;
};

// Row length of the packed V^T and its size in bytes.
inline int attention_l_pad(int L) { return (L + 127) / 128 * 128; }
inline size_t attention_vt_bytes(const tsa_problem_t* p) {
  const size_t elt = p->dtype == TSA_DTYPE_BF16 ? 2 : 4;
  return (size_t)p->B * p->H * (size_t)(p->d + 1) * (size_t)attention_l_pad(p->L) * elt;
}

hipError_t launch_attention_bf16(const AttnLaunch& a);
hipError_t launch_attention_f32(const AttnLaunch& a);

}  // namespace tsa
