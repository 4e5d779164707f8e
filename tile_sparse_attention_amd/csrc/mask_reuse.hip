// Difference of two keep-bitmaps, for reusing a predicted mask across
// denoising steps (gfx950, wave64).
//
// FG-Attn ("FG-Attn: Leveraging Fine-Grained Sparse Attention in Video
// Diffusion Models", section Abstract) decides per M x N tile whether its
// scores are computed.  How far two masks of the same problem are apart is
// the number of tiles whose decision differs: per bitmap row (b, h, i) the
// popcount of (a XOR b) over key tiles j < T_k (padding bits past T_k are not
// decisions), and per head the sum over its rows.
//
// Both passes stream their inputs once and are bound by HBM bandwidth:
//   * diff_rows_kernel: one wave per four bitmap rows; lanes read consecutive
//     words (16 bytes per lane when rows are 16-byte aligned), the last word
//     is masked to the row's T_k bits, and a wave reduction gives each count.
//   * diff_heads_kernel: one work-group per head sums its rows' counts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsa.h"
#include "tsa_device.h"

namespace tsa {

namespace {

// Rows per wave: the loads of all of them are in flight before the first
// reduction.
constexpr int kRowsPerWave = 4;

template <bool VEC>
__global__ __launch_bounds__(256) void diff_rows_kernel(const uint32_t* __restrict__ a,
                                                        const uint32_t* __restrict__ b, long long rows,
                                                        int words, uint32_t last_mask,
                                                        int64_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  // work-groups of 4 waves x kRowsPerWave rows, stepping with the grid's stride
  for (long long blk = blockIdx.x; blk * 4 * kRowsPerWave < rows; blk += gridDim.x) {
    const long long r0 = (blk * 4 + (threadIdx.x >> 6)) * kRowsPerWave;
    int cnt[kRowsPerWave];
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
      cnt[k] = 0;
      const long long r = r0 + k;
      if (r >= rows) continue;
      const uint32_t* ra = a + r * words;
      const uint32_t* rb = b + r * words;
      if constexpr (VEC) {
        // words % 4 == 0: 16-byte aligned rows, four words per lane per step
        for (int w = 4 * lane; w < words; w += 256) {
          const uint4 x = *reinterpret_cast<const uint4*>(ra + w);
          const uint4 y = *reinterpret_cast<const uint4*>(rb + w);
          uint32_t z3 = x.w ^ y.w;
          if (w + 4 == words) z3 &= last_mask;
          cnt[k] += __builtin_popcount(x.x ^ y.x) + __builtin_popcount(x.y ^ y.y) +
                    __builtin_popcount(x.z ^ y.z) + __builtin_popcount(z3);
        }
      } else {
        for (int w = lane; w < words; w += 64) {
          uint32_t x = ra[w] ^ rb[w];
          if (w == words - 1) x &= last_mask;
          cnt[k] += __builtin_popcount(x);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
      int c = cnt[k];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o);
      if (lane == 0 && r0 + k < rows) out[r0 + k] = c;
    }
  }
}

__global__ __launch_bounds__(256) void diff_heads_kernel(const int64_t* __restrict__ row_counts, int T_q,
                                                         int64_t* __restrict__ out) {
  __shared__ long long part[4];
  const long long* rc = reinterpret_cast<const long long*>(row_counts) + (size_t)blockIdx.x * T_q;
  long long s = 0;
  for (int i = threadIdx.x; i < T_q; i += 256) s += rc[i];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

}  // namespace

hipError_t launch_mask_diff(const tsa_problem_t* p, const uint32_t* a, const uint32_t* b, int64_t* rows_out,
                            int64_t* heads_out, hipStream_t stream) {
  const int T_q = (p->L + p->M - 1) / p->M;
  const int T_k = (p->L + p->N - 1) / p->N;
  const int words = (T_k + 31) / 32;
  const long long rows = (long long)p->B * p->H * T_q;
  const uint32_t last_mask = (T_k & 31) ? ((1u << (T_k & 31)) - 1u) : 0xffffffffu;
  const unsigned blocks = stride_blocks(rows, 4 * kRowsPerWave);
  if (words % 4 == 0)
    hipLaunchKernelGGL(diff_rows_kernel<true>, dim3(blocks), dim3(256), 0, stream, a, b, rows, words, last_mask,
                       rows_out);
  else
    hipLaunchKernelGGL(diff_rows_kernel<false>, dim3(blocks), dim3(256), 0, stream, a, b, rows, words,
                       last_mask, rows_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || heads_out == nullptr) return e;
  hipLaunchKernelGGL(diff_heads_kernel, dim3((unsigned)(p->B * p->H)), dim3(256), 0, stream, rows_out, T_q,
                     heads_out);
  return hipGetLastError();
}

}  // namespace tsa
