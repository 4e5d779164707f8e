// bf16 instances of the tile-sparse attention forward kernel.
#include "attention_fwd_inst.h"

namespace tsa {
hipError_t launch_attention_bf16(const AttnLaunch& a) { return launch_attn_t<bf16_t>(a); }
}  // namespace tsa
