// Mask compaction: keep-bitmap rows -> CSR lists of kept key tiles.
//
// FG-Attn ("FG-Attn: Leveraging Fine-Grained Sparse Attention in Video
// Diffusion Models", section Abstract) makes one skip decision per M x N tile;
// this turns each query-tile row of decisions into the ascending list of kept
// key tiles.  Three passes, all bandwidth-bound scans of the bitmap:
//   1. count:  one wave per row sums the popcounts of its words (padding bits
//              past T_k cleared) and each work-group sums its rows;
//   2. scan:   one work-group turns the per-group sums into int64 offsets;
//   3. fill:   one wave per row writes row_ptr and walks its row in 64-tile
//              windows with wave_compact64, the same routine the attention
//              kernel uses on the fly, clipping writes at col_capacity.
#include "tsa_device.h"
#include "tsa.h"

namespace tsa {

constexpr int kRowsPerGroup = 4;  // one wave per row, 4 waves per work-group

__global__ __launch_bounds__(256) void compact_count_kernel(const uint32_t* __restrict__ mask,
                                                            long long rows, int words, int T_k,
                                                            int32_t* __restrict__ counts,
                                                            long long* __restrict__ group_sums) {
  __shared__ int part[kRowsPerGroup];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * kRowsPerGroup + wave;
  int cnt = 0;
  if (row < rows) {
    const uint32_t* r = mask + row * (long long)words;
    for (int w = lane; w < words; w += 64) {
      uint32_t x = r[w];
      const int valid = T_k - 32 * w;
      if (valid < 32) x &= (1u << valid) - 1u;
      cnt += __builtin_popcount(x);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off);
    if (lane == 0) counts[row] = cnt;
  }
  if (lane == 0) part[wave] = row < rows ? cnt : 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long s = 0;
    for (int i = 0; i < kRowsPerGroup; ++i) s += part[i];
    group_sums[blockIdx.x] = s;
  }
}

// Exclusive scan of `n` int64 values in place by a single work-group of 1024
// threads; total[0] receives the sum.
__global__ __launch_bounds__(1024) void scan_groups_kernel(long long* __restrict__ v, long long n,
                                                           long long* __restrict__ total) {
  __shared__ long long part[1024];
  const int t = threadIdx.x;
  const long long per = (n + 1023) / 1024;
  const long long b = t * per, e = b + per < n ? b + per : n;
  long long s = 0;
  for (long long i = b; i < e; ++i) s += v[i];
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // Hillis-Steele inclusive scan of the parts
    const long long x = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += x;
    __syncthreads();
  }
  long long run = t > 0 ? part[t - 1] : 0;
  for (long long i = b; i < e; ++i) {
    const long long x = v[i];
    v[i] = run;
    run += x;
  }
  if (t == 1023) total[0] = part[1023];
}

__global__ __launch_bounds__(256) void compact_fill_kernel(
    const uint32_t* __restrict__ mask, long long rows, int words, int T_k,
    const int32_t* __restrict__ counts, const long long* __restrict__ group_offsets,
    const long long* __restrict__ total, long long* __restrict__ row_ptr,
    int32_t* __restrict__ col_idx, long long col_capacity) {
  const int wave = wave_uniform(threadIdx.x >> 6);
  const long long row = (long long)blockIdx.x * kRowsPerGroup + wave;
  if (row >= rows) return;
  long long start = group_offsets[blockIdx.x];
  for (int i = 0; i < wave; ++i) start += counts[row - wave + i];
  if (lane_id() == 0) {
    row_ptr[row] = start;
    if (row == rows - 1) row_ptr[rows] = total[0];
  }
  const uint32_t* r = mask + row * (long long)words;
  uint32_t done = 0;
  for (int first = 0; first < T_k; first += 64) {
    const uint64_t bits = row_bits(r, first, 64, T_k);
    done += wave_compact64(bits, first, done, [&](uint32_t pos, int val) {
      const long long at = start + (long long)pos;
      if (at < col_capacity) col_idx[at] = val;
    });
  }
}

hipError_t launch_mask_compact(const tsa_problem_t* p, const uint32_t* mask, int64_t* row_ptr,
                               int32_t* col_idx, int64_t col_capacity, void* workspace,
                               hipStream_t stream) {
  const int T_q = (p->L + p->M - 1) / p->M;
  const int T_k = (p->L + p->N - 1) / p->N;
  const int words = (T_k + 31) / 32;
  const long long rows = (long long)p->B * p->H * T_q;
  const long long groups = (rows + kRowsPerGroup - 1) / kRowsPerGroup;
  char* ws = static_cast<char*>(workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(ws);
  size_t off = ((size_t)rows * sizeof(int32_t) + 255) & ~(size_t)255;
  long long* gsum = reinterpret_cast<long long*>(ws + off);
  off += ((size_t)groups * sizeof(long long) + 255) & ~(size_t)255;
  long long* total = reinterpret_cast<long long*>(ws + off);

  hipLaunchKernelGGL(compact_count_kernel, dim3((unsigned)groups), dim3(256), 0, stream, mask, rows,
                     words, T_k, counts, gsum);
  hipLaunchKernelGGL(scan_groups_kernel, dim3(1), dim3(1024), 0, stream, gsum, groups, total);
  hipLaunchKernelGGL(compact_fill_kernel, dim3((unsigned)groups), dim3(256), 0, stream, mask, rows,
                     words, T_k, counts, gsum, total, reinterpret_cast<long long*>(row_ptr), col_idx,
                     (long long)col_capacity);
  return hipGetLastError();
}

size_t mask_compact_workspace(const tsa_problem_t* p) {
  const long long T_q = (p->L + p->M - 1) / p->M;
  const long long rows = (long long)p->B * p->H * T_q;
  const long long groups = (rows + kRowsPerGroup - 1) / kRowsPerGroup;
  size_t off = ((size_t)rows * sizeof(int32_t) + 255) & ~(size_t)255;
  off += ((size_t)groups * sizeof(long long) + 255) & ~(size_t)255;
  return off + 256;
}

}  // namespace tsa
