// FP8 instances of the octet kernel (N >= 8) and of the key kernel (N < 8):
// Q and K as e4m3 bytes with per-tile scales, scores on the 16x16x128 FP8
// matrix cores; V, P and O stay bf16.  d = 128.
#include "attention_fwd_inst.h"

namespace tsa {

hipError_t launch_attention_fp8(const AttnLaunch& a) {
  switch (a.p->N) {
    case 1: return launch_attn_key<128, 1, true>(a);
    case 2: return launch_attn_key<128, 2, true>(a);
    case 4: return launch_attn_key<128, 4, true>(a);
    case 8: return launch_attn_oct<128, 8, true>(a);
    case 16: return launch_attn_oct<128, 16, true>(a);
    case 32: return launch_attn_oct<128, 32, true>(a);
    case 64: return launch_attn_oct<128, 64, true>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tsa
