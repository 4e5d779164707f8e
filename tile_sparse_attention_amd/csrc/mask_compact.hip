// Mask compaction: keep-bitmap rows -> CSR lists of kept key tiles.
//
// FG-Attn ("FG-Attn: Leveraging Fine-Grained Sparse Attention in Video
// Diffusion Models", section Abstract) makes one skip decision per M x N tile;
// this turns each query-tile row of decisions into the ascending list of kept
// key tiles.  Three passes, all bandwidth-bound scans of the bitmap:
//   1. count:  one wave per row sums the popcounts of its words (padding bits
//              past T_k cleared) and each work-group sums its 16 rows;
//   2. scan:   one work-group turns the per-group sums into int64 offsets;
//   3. fill:   one wave per row writes row_ptr, then takes its row 64 words
//              at a time: one coalesced load (a word per lane), a wave prefix
//              sum of the words' popcounts for each lane's first slot, each
//              lane's kept tiles into the wave's LDS staging area in
//              ascending order, and from there contiguous coalesced stores,
//              clipped at col_capacity.  A row that starts at or past
//              col_capacity (a count-only call) reads no bits at all.
#include "tsa_device.h"
#include "tsa.h"

namespace tsa {

constexpr int kRowsPerGroup = 16;  // rows per count work-group (one wave each) and per scan entry
constexpr int kFillWaves = 4;      // rows per fill work-group (one wave each)

__global__ __launch_bounds__(64 * kRowsPerGroup) void compact_count_kernel(const uint32_t* __restrict__ mask,
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

// Orders this wave's LDS accesses on either side of it (a wave's LDS
// operations complete in issue order; this keeps the compiler from moving
// them across).
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(64 * kFillWaves) void compact_fill_kernel(
    const uint32_t* __restrict__ mask, long long rows, int words, int T_k,
    const int32_t* __restrict__ counts, const long long* __restrict__ group_offsets,
    const long long* __restrict__ total, long long* __restrict__ row_ptr,
    int32_t* __restrict__ col_idx, long long col_capacity) {
  __shared__ int32_t stage[kFillWaves][64 * 32];  // a block's kept tiles, per wave
  const int wave = wave_uniform(threadIdx.x >> 6);
  const long long row = (long long)blockIdx.x * kFillWaves + wave;
  if (row >= rows) return;
  // the row's count group's offset plus the counts of the group's earlier rows
  const long long grp = row / kRowsPerGroup, first = grp * kRowsPerGroup;
  long long start = group_offsets[grp];
  for (long long i = first; i < row; ++i) start += counts[i];
  if (lane_id() == 0) {
    row_ptr[row] = start;
    if (row == rows - 1) row_ptr[rows] = total[0];
  }
  if (start >= col_capacity) return;
  const uint32_t* r = mask + row * (long long)words;
  const int lane = lane_id();
  int32_t* st = stage[wave];
  long long base = start;  // output slot of the block's first kept tile
  // each block's words are loaded while the previous block is written
  uint32_t xn = lane < words ? r[lane] : 0u;
  for (int w0 = 0; w0 < words && base < col_capacity; w0 += 64) {
    const int w = w0 + lane;
    uint32_t x = xn;
    xn = w + 64 < words ? r[w + 64] : 0u;
    if (w < words) {
      const int valid = T_k - 32 * w;  // 1..32 in the last word
      if (valid < 32) x &= (1u << valid) - 1u;
    }
    const int c = __builtin_popcount(x);
    int incl = c;  // inclusive prefix sum of the popcounts over the lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int at = incl - c;
    while (x != 0u) {
      const int b = __builtin_ctz(x);
      x &= x - 1u;
      st[at++] = 32 * w + b;
    }
    wave_sync_lds();  // the staging writes of every lane precede the reads
    const int total_blk = __shfl(incl, 63);
    for (int j = lane; j < total_blk; j += 64)
      if (base + j < col_capacity) col_idx[base + j] = st[j];
    wave_sync_lds();  // ... and the reads precede the next block's writes
    base += total_blk;
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

  const long long fill_groups = (rows + kFillWaves - 1) / kFillWaves;
  hipLaunchKernelGGL(compact_count_kernel, dim3((unsigned)groups), dim3(64 * kRowsPerGroup), 0, stream, mask,
                     rows, words, T_k, counts, gsum);
  hipLaunchKernelGGL(scan_groups_kernel, dim3(1), dim3(1024), 0, stream, gsum, groups, total);
  hipLaunchKernelGGL(compact_fill_kernel, dim3((unsigned)fill_groups), dim3(64 * kFillWaves), 0, stream, mask, rows,
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
