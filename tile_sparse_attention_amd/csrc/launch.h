// Kernel launchers called by the C ABI layer (api.hip).  Each returns the
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
  void* workspace;  // packed V^T, then chunk bitmaps: attention_workspace_bytes()
  hipStream_t stream;
  // FP8 scores: q and k hold e4m3 bytes with these scales (null otherwise)
  const float* q_scale = nullptr;
  const float* k_scale = nullptr;
  // when set, recorded on `stream` right before and right after the attention
  // kernel(s) proper (not the V^T pack or the chunk pre-pass)
  hipEvent_t ev_start = nullptr;
  hipEvent_t ev_stop = nullptr;
};

inline void mark_event(hipEvent_t e, hipStream_t s) {
  if (e != nullptr) (void)hipEventRecord(e, s);
}

// Row length of the packed V^T and its size in bytes.
inline int attention_l_pad(int L) { return (L + 127) / 128 * 128; }
inline size_t attention_vt_bytes(const tsa_problem_t* p) {
  const size_t elt = p->dtype == TSA_DTYPE_BF16 ? 2 : 4;
  return (size_t)p->B * p->H * (size_t)(p->d + 1) * (size_t)attention_l_pad(p->L) * elt;
}

// Chunk skipping (bf16, N >= 8, at most 2048 chunks of 128 keys): per
// work-group of 256 query rows, a 64-word bitmap of the key chunks any of
// its rows keeps a tile of and a flag word (1: skipping would pay off for
// it), then one count of flagged work-groups.
constexpr int kChunkKeys = 128, kRowsPerGroup = 256, kMaxChunks = 2048, kNeedWords = kMaxChunks / 32;
inline bool attention_skips_chunks(const tsa_problem_t* p) {
  return p->dtype == TSA_DTYPE_BF16 && p->N >= 8 && (p->L + kChunkKeys - 1) / kChunkKeys <= kMaxChunks;
}
inline size_t attention_groups(const tsa_problem_t* p) {
  return (size_t)p->B * p->H * (size_t)((p->L + kRowsPerGroup - 1) / kRowsPerGroup);
}
inline size_t attention_need_offset(const tsa_problem_t* p) {
  return (attention_vt_bytes(p) + 255) / 256 * 256;
}
inline size_t attention_workspace_bytes(const tsa_problem_t* p) {
  if (!attention_skips_chunks(p)) return attention_vt_bytes(p);
  return attention_need_offset(p) + (attention_groups(p) * (kNeedWords + 1) + 1) * sizeof(uint32_t);
}

// Backward (bf16): the workspace holds, per (b, h) and 128-row chunk, the
// chunk's 128 lse2 values and 128 D values (fp32).
struct BwdLaunch {
  const tsa_problem_t* p;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  const uint32_t* mask;
  float scale;
  void* dq;
  void* dk;
  void* dv;
  void* workspace;
  hipStream_t stream;
};
inline size_t attention_bwd_workspace_bytes(const tsa_problem_t* p) {
  return (size_t)p->B * p->H * (size_t)((p->L + 127) / 128) * 256 * sizeof(float);
}
hipError_t launch_attention_bwd(const BwdLaunch& a);

hipError_t launch_attention_bf16(const AttnLaunch& a);
hipError_t launch_attention_fp8(const AttnLaunch& a);
hipError_t launch_quantize_qk_fp8(const tsa_problem_t* p, const void* q, const void* k, uint8_t* q8,
                                  float* q_scale, uint8_t* k8, float* k_scale, hipStream_t stream);
hipError_t launch_attention_f32(const AttnLaunch& a);

}  // namespace tsa
