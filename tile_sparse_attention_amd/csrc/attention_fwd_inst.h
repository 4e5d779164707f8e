// Instantiation table of the attention kernel for one element type.
#pragma once

#include "attention_fwd_impl.h"
#include "attention_fwd_keys.h"
#include "attention_fwd_octet.h"
#include "launch.h"

namespace tsa {

inline AttnParams attn_params(const AttnLaunch& a, int rows_per_block) {
  const tsa_problem_t& pr = *a.p;
  AttnParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.vt = a.workspace;
  p.mask = a.mask;
  p.o = a.o;
  p.lse = a.lse;
  p.H = pr.H;
  p.L = pr.L;
  p.M = pr.M;
  p.T_q = (pr.L + pr.M - 1) / pr.M;
  p.T_k = (pr.L + pr.N - 1) / pr.N;
  p.words = (p.T_k + 31) / 32;
  p.L_pad = attention_l_pad(pr.L);
  p.n_qblocks = (pr.L + rows_per_block - 1) / rows_per_block;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.need = nullptr;
  p.need_flag = nullptr;
  p.need_count = nullptr;
  p.q_scale = a.q_scale;
  p.k_scale = a.k_scale;
  return p;
}

template <typename T, int D>
void launch_vt_pack(const AttnLaunch& a, const AttnParams& p) {
  // a block per 64 keys of each (b, h), on the x dimension only; any problem
  // whose tensors fit in memory stays below 2^31 blocks
  const long long blocks = (long long)(p.L_pad / 64) * a.p->B * a.p->H;
  hipLaunchKernelGGL((vt_pack_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, a.stream,
                     static_cast<const T*>(a.v), static_cast<T*>(a.workspace), a.p->L, p.L_pad);
}

template <typename T, int D, int N, int KC, int W, int TPW>
hipError_t launch_attn_cfg(const AttnLaunch& a) {
  const AttnParams p = attn_params(a, 16 * TPW * W);
  const long long blocks = (long long)a.p->B * a.p->H * p.n_qblocks;
  launch_vt_pack<T, D>(a, p);
  mark_event(a.ev_start, a.stream);
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, N, KC, W, TPW>), dim3((unsigned)blocks), dim3(64 * W), 0,
                     a.stream, p);
  mark_event(a.ev_stop, a.stream);
  return hipGetLastError();
}

// bf16 with key tiles of N >= 8: the octet-packing kernel.
// With chunk skipping (at most kMaxChunks chunks), chunk_need_kernel first
// sorts the work-groups into those that need nearly every chunk (run by the
// plain kernel) and the rest (run by the skipping kernel).
template <int D, int N, bool F8 = false>
hipError_t launch_attn_oct(const AttnLaunch& a) {
  using C = OctCfg<D, N, F8>;
  AttnParams p = attn_params(a, C::ROWS);
  const long long blocks = (long long)a.p->B * a.p->H * p.n_qblocks;
  launch_vt_pack<bf16_t, D>(a, p);
  if (!attention_skips_chunks(a.p)) {
    mark_event(a.ev_start, a.stream);
    hipLaunchKernelGGL((attn_oct_kernel<D, N, false, F8>), dim3((unsigned)blocks), dim3(64 * C::W), 0,
                       a.stream, p);
    mark_event(a.ev_stop, a.stream);
    return hipGetLastError();
  }
  uint32_t* need = reinterpret_cast<uint32_t*>(static_cast<char*>(a.workspace) +
                                               attention_need_offset(a.p));
  uint32_t* flag = need + attention_groups(a.p) * kNeedWords;
  uint32_t* count = flag + attention_groups(a.p);
  p.need = need;
  p.need_flag = flag;
  p.need_count = count;
  hipLaunchKernelGGL(zero_word_kernel<uint32_t>, dim3(1), dim3(64), 0, a.stream, count);
  hipLaunchKernelGGL((chunk_need_kernel<N>), dim3((unsigned)blocks), dim3(256), 0, a.stream, p, need, flag,
                     count);
  mark_event(a.ev_start, a.stream);
  hipLaunchKernelGGL((attn_oct_kernel<D, N, false, F8>), dim3((unsigned)blocks), dim3(64 * C::W), 0, a.stream,
                     p);
  hipLaunchKernelGGL((attn_oct_kernel<D, N, true, F8>), dim3((unsigned)blocks), dim3(64 * C::W), 0, a.stream,
                     p);
  mark_event(a.ev_stop, a.stream);
  return hipGetLastError();
}

// bf16 with key tiles of N < 8: the key-packing kernel (V read as rows, no
// V^T workspace).
template <int D, int N, bool F8 = false>
hipError_t launch_attn_key(const AttnLaunch& a) {
  using C = KeyCfg<D, N, F8>;
  const AttnParams p = attn_params(a, C::ROWS);
  const long long blocks = (long long)a.p->B * a.p->H * p.n_qblocks;
  mark_event(a.ev_start, a.stream);
  hipLaunchKernelGGL((attn_key_kernel<D, N, F8>), dim3((unsigned)blocks), dim3(64 * C::W), 0, a.stream, p);
  mark_event(a.ev_stop, a.stream);
  return hipGetLastError();
}

// Chunk size KC, waves per work-group W and 16-row tiles per wave TPW per
// (element type, head dim, N): the double-buffered K and V^T chunks stay
// within the 160 KB of LDS, and every variant fits the register file without
// spilling (checked at build time).  Sixteen one-tile waves (four per SIMD)
// hide latency best; the N < 4 gathers need the larger budget of eight
// two-tile waves.
template <typename T, int D, int N> struct AttnShape;
template <int N> struct AttnShape<bf16_t, 128, N> {
  static constexpr int KC = 128, W = N >= 4 ? 16 : 8, TPW = N >= 4 ? 1 : 2;
};
template <int N> struct AttnShape<bf16_t, 64, N> { static constexpr int KC = 128, W = 16, TPW = 1; };
template <int N> struct AttnShape<float, 128, N> { static constexpr int KC = 64, W = 8, TPW = 2; };
template <int N> struct AttnShape<float, 64, N> { static constexpr int KC = 64, W = 4, TPW = 2; };

template <typename T, int D, int N>
hipError_t launch_attn_n(const AttnLaunch& a) {
  if constexpr (sizeof(T) == 2 && N >= 8) {
    return launch_attn_oct<D, N>(a);
  } else if constexpr (sizeof(T) == 2) {
    return launch_attn_key<D, N>(a);
  } else {
    using S = AttnShape<T, D, N>;
    return launch_attn_cfg<T, D, N, S::KC, S::W, S::TPW>(a);
  }
}

template <typename T, int D>
hipError_t launch_attn_d(const AttnLaunch& a) {
  switch (a.p->N) {
    case 1: return launch_attn_n<T, D, 1>(a);
    case 2: return launch_attn_n<T, D, 2>(a);
    case 4: return launch_attn_n<T, D, 4>(a);
    case 8: return launch_attn_n<T, D, 8>(a);
    case 16: return launch_attn_n<T, D, 16>(a);
    case 32: return launch_attn_n<T, D, 32>(a);
    case 64: return launch_attn_n<T, D, 64>(a);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_attn_t(const AttnLaunch& a) {
  switch (a.p->d) {
    case 64: return launch_attn_d<T, 64>(a);
    case 128: return launch_attn_d<T, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tsa
