// fp32 instances of the tile-sparse attention forward kernel.
#include "attention_fwd_inst.h"

namespace tsa {
hipError_t launch_attention_f32(const AttnLaunch& a) { return launch_attn_t<float>(a); }
}  // namespace tsa
