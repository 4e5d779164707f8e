// Synthetic keep-bitmap generator (workload support, not the attention
// method): a thread per output word (stepping through the words with the
// grid's stride) evaluates 32 tiles of the counter-based SplitMix64 recipe
// described in tsa_workload.h.
#include "tsa_device.h"
#include "tsa.h"
#include "tsa_workload.h"

namespace tsa {

__device__ __forceinline__ uint64_t splitmix64_at(uint64_t state0, uint64_t ctr) {
  uint64_t z = state0 + (ctr + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ __launch_bounds__(256) void maskgen_hash_kernel(uint32_t* __restrict__ out,
                                                           long long total_words, int H, int L,
                                                           int M, int N, int T_q, int T_k,
                                                           int words, tsa_maskgen_params_t g) {
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total_words;
       idx += (long long)gridDim.x * 256) {
    const int w = (int)(idx % words);
    const long long row = idx / words;            // (b*H + h)*T_q + i
    const int i = (int)(row % T_q);
    const int r0 = i * M;
    const int r1 = r0 + M < L ? r0 + M : L;
    const int fq = g.frame_tokens > 0 ? r0 / g.frame_tokens : 0;
    uint32_t bits = 0;
    for (int t = 0; t < 32; ++t) {
      const int j = 32 * w + t;
      if (j >= T_k) break;
      const uint64_t z = splitmix64_at(g.state0, (uint64_t)row * (uint64_t)T_k + (uint64_t)j);
      uint32_t thr = g.thr_near;
      if (g.frame_tokens > 0) {
        const int fk = (int)(((long long)j * N) / g.frame_tokens);
        const int df = fk > fq ? fk - fq : fq - fk;
        if (df > g.frame_radius) thr = g.thr_far;
      }
      bool keep = (uint32_t)(z >> 40) < thr;
      if (g.force_diag) {
        const int c0 = j * N;
        const int c1 = c0 + N < L ? c0 + N : L;
        keep = keep || (c0 < r1 && r0 < c1);
      }
      bits |= (uint32_t)keep << t;
    }
    out[idx] = bits;
  }
}

hipError_t launch_maskgen_hash(const tsa_problem_t* p, const tsa_maskgen_params_t* g,
                               uint32_t* out, hipStream_t stream) {
  const int T_q = (p->L + p->M - 1) / p->M;
  const int T_k = (p->L + p->N - 1) / p->N;
  const int words = (T_k + 31) / 32;
  const long long total = (long long)p->B * p->H * T_q * words;
  hipLaunchKernelGGL(maskgen_hash_kernel, dim3(stride_blocks(total, 256)), dim3(256), 0,
                     stream, out, total, p->H, p->L, p->M, p->N, T_q, T_k, words, *g);
  return hipGetLastError();
}

// Structured patterns (tsa_workload.h): one thread per output word, closed
// forms per tile.
struct StructuredArgs {
  tsa_structured_params_t s;
  int8_t pattern[TSA_MAX_PATTERN_HEADS];
};

__device__ __forceinline__ bool ranges_meet(long long a0, long long a1, long long b0, long long b1) {
  return a0 <= b1 && b0 <= a1;  // inclusive ranges
}

__global__ __launch_bounds__(256) void maskgen_structured_kernel(uint32_t* __restrict__ out,
                                                                 long long total_words, int H, int L,
                                                                 int M, int N, int T_q, int T_k,
                                                                 int words, StructuredArgs g) {
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total_words;
       idx += (long long)gridDim.x * 256) {
    const int w = (int)(idx % words);
    const long long row = idx / words;  // (b*H + h)*T_q + i
    const int i = (int)(row % T_q);
    const int h = (int)((row / T_q) % H);
    const int pat = g.pattern[h];
    const long long q0 = (long long)i * M;
    const long long q1 = (q0 + M < L ? q0 + M : L) - 1;
    uint32_t bits = 0;
    for (int t = 0; t < 32; ++t) {
      const int j = 32 * w + t;
      if (j >= T_k) break;
      const long long k0 = (long long)j * N;
      const long long k1 = (k0 + N < L ? k0 + N : L) - 1;
      bool keep = false;
      if (pat == TSA_PATTERN_DENSE) {
        keep = true;
      } else if (pat == TSA_PATTERN_DIAGONAL) {
        // some k in [k0, k1] within width of some q in [q0, q1]
        keep = ranges_meet(k0, k1, q0 - g.s.diag_width, q1 + g.s.diag_width);
      } else if (pat == TSA_PATTERN_MULTI_DIAGONAL) {
        for (int d = -g.s.reach; d <= g.s.reach && !keep; ++d) {
          const long long sft = (long long)d * g.s.frame_tokens;
          keep = ranges_meet(k0, k1, q0 + sft - g.s.band_width, q1 + sft + g.s.band_width);
        }
      } else if (pat == TSA_PATTERN_VERTICAL_STRIPE) {
        const long long P = g.s.stripe_period;
        if (g.s.stripe_width > 0) {
          const long long r = k0 % P;  // first stripe key at or after k0
          const long long first = r < g.s.stripe_width ? k0 : k0 + (P - r);
          keep = first <= k1;
        }
      }
      bits |= (uint32_t)keep << t;
    }
    out[idx] = bits;
  }
}

hipError_t launch_maskgen_structured(const tsa_problem_t* p, const tsa_structured_params_t* s,
                                     const int32_t* head_pattern, uint32_t* out, hipStream_t stream) {
  const int T_q = (p->L + p->M - 1) / p->M;
  const int T_k = (p->L + p->N - 1) / p->N;
  const int words = (T_k + 31) / 32;
  const long long total = (long long)p->B * p->H * T_q * words;
  StructuredArgs g;
  g.s = *s;
  for (int h = 0; h < TSA_MAX_PATTERN_HEADS; ++h) g.pattern[h] = h < p->H ? (int8_t)head_pattern[h] : 0;
  hipLaunchKernelGGL(maskgen_structured_kernel, dim3(stride_blocks(total, 256)), dim3(256), 0,
                     stream, out, total, p->H, p->L, p->M, p->N, T_q, T_k, words, g);
  return hipGetLastError();
}

}  // namespace tsa
