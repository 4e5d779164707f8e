// Mask compaction: keep-bitmap rows -> CSR lists of kept key tiles.
//
// FG-Attn ("FG-Attn: Leveraging Fine-Grained Sparse Attention in Video
// Diffusion Models", section Abstract) makes one skip decision per M x N tile;
// this turns each query-tile row of decisions into the ascending list of kept
// key tiles.  Three passes, all bandwidth-bound scans of the bitmap (the
// count and fill work-groups step through their row groups with the grid's
// stride, so any number of rows fits one launch):
//   1. count:  one wave per row sums the popcounts of its words (padding bits
//              past T_k cleared) and each work-group sums its 16 rows;
//   2. scan:   one work-group turns the per-group sums into int64 offsets;
//   3. fill:   one wave per row writes row_ptr, then takes its row 64 words
//              at a time: a word per lane (loaded 16 blocks at a time, one
//              such super-block ahead), a wave prefix sum of the words'
//              popcounts for each lane's first slot, each lane's kept tiles
//              into the wave's LDS staging area in ascending order (placed at
//              the output's alignment), and from there 16-byte stores of
//              aligned runs, clipped at col_capacity.  A row that starts at or
//              past col_capacity (a count-only call) reads no bits at all.
#include "tsa_device.h"
#include "tsa.h"

namespace tsa {

constexpr int kRowsPerGroup = 16;  // rows per count work-group (one wave each) and per scan entry
constexpr int kFillWaves = 4;      // rows per fill work-group (one wave each)
constexpr int kSuperBlock = 16;    // 64-word blocks of a row loaded together by the fill

__global__ __launch_bounds__(64 * kRowsPerGroup) void compact_count_kernel(const uint32_t* __restrict__ mask,
                                                            long long rows, int words, int T_k,
                                                            int32_t* __restrict__ counts,
                                                            long long* __restrict__ group_sums) {
  __shared__ int part[kRowsPerGroup];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const long long groups = (rows + kRowsPerGroup - 1) / kRowsPerGroup;
  for (long long grp = blockIdx.x; grp < groups; grp += gridDim.x) {
    const long long row = grp * kRowsPerGroup + wave;
    int cnt = 0;
    if (row < rows) {
      const uint32_t* r = mask + row * (long long)words;
      // eight independent loads in flight per lane: the row's words are read
      // at the memory system's rate, not at one load latency per 256 bytes
      for (int w0 = 0; w0 < words; w0 += 64 * 8) {
        uint32_t x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int w = w0 + 64 * u + lane;
          x[u] = w < words ? r[w] : 0u;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int w = w0 + 64 * u + lane;
          const int valid = T_k - 32 * w;
          if (valid < 32) x[u] &= valid > 0 ? (1u << valid) - 1u : 0u;
          cnt += __builtin_popcount(x[u]);
        }
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
      group_sums[grp] = s;
    }
    __syncthreads();  // part is rewritten for the next group
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

// One row of the fill, by one wave; st: the wave's LDS staging area.
__device__ __forceinline__ void fill_row(const uint32_t* __restrict__ mask, long long row, long long rows,
                                         int words, int T_k, const int32_t* __restrict__ counts,
                                         const long long* __restrict__ group_offsets,
                                         const long long* __restrict__ total, long long* __restrict__ row_ptr,
                                         int32_t* __restrict__ col_idx, long long col_capacity, int32_t* st) {
  const uint32_t* r = mask + row * (long long)words;
  const int lane = lane_id();
  // The row's words come kSuperBlock 64-word blocks at a time, a word per
  // lane per block, loaded one super-block ahead.  The first super-block is
  // requested before the row's offset is known, so that the two loads'
  // latencies overlap; a count-only call (capacity 0) reads no words.
  const int nblk = (words + 63) >> 6;
  uint32_t xn[kSuperBlock];
  if (col_capacity > 0) {
#pragma unroll
    for (int u = 0; u < kSuperBlock; ++u) {
      const int w = 64 * u + lane;
      xn[u] = w < words ? r[w] : 0u;
    }
  }
  // the row's count group's offset plus the counts of the group's earlier
  // rows (lane i holds the count of the group's row i; one vector load)
  const long long grp = row / kRowsPerGroup, first = grp * kRowsPerGroup;
  const int li = lane;
  int before = li < (int)(row - first) ? counts[first + li] : 0;
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) before += __shfl_xor(before, off);  // lanes 0..15 hold all
  long long start = group_offsets[grp] + (long long)__shfl(before, 0);
  if (lane_id() == 0) {
    row_ptr[row] = start;
    if (row == rows - 1) row_ptr[rows] = total[0];
  }
  if (start >= col_capacity) return;
  long long base = start;  // output slot of the block's first kept tile
  // A vector-memory wait also waits for the stores issued before it, so
  // waiting once per super-block instead of once per block lets a block's
  // stores overlap the next blocks' expansion.
  for (int b0 = 0; b0 < nblk && base < col_capacity; b0 += kSuperBlock) {
    uint32_t xc[kSuperBlock];
#pragma unroll
    for (int u = 0; u < kSuperBlock; ++u) xc[u] = xn[u];
    if (b0 + kSuperBlock < nblk) {
#pragma unroll
      for (int u = 0; u < kSuperBlock; ++u) {
        const int w = 64 * (b0 + kSuperBlock + u) + lane;
        xn[u] = w < words ? r[w] : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < kSuperBlock; ++u) {
      if (b0 + u >= nblk || base >= col_capacity) break;
      const int w = 64 * (b0 + u) + lane;
      uint32_t x = xc[u];
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
      // staged at the output's alignment: stage slot a + s holds output slot
      // base + s, with a = (address of col_idx[base] / 4) mod 4, so every four
      // stage slots 4m..4m+3 are one 16-byte-aligned run of col_idx
      const int a = (int)((reinterpret_cast<uintptr_t>(col_idx + base) >> 2) & 3);
      int at = a + incl - c;
      while (x != 0u) {
        const int bb = __builtin_ctz(x);
        x &= x - 1u;
        st[at++] = 32 * w + bb;
      }
      wave_sync_lds();  // the staging writes of every lane precede the reads
      const int total_blk = __shfl(incl, 63);
      const long long g0 = base - a;  // output slot of stage slot 0 (16-byte aligned)
      const int end = a + total_blk;  // stage slots a .. end-1 are this block's
      for (int m = lane; 4 * m < end; m += 64) {
        const int s0 = 4 * m;
        const long long gs = g0 + s0;
        if (s0 >= a && s0 + 4 <= end && gs + 4 <= col_capacity) {
          const int4 v = *reinterpret_cast<const int4*>(&st[s0]);
          *reinterpret_cast<int4*>(col_idx + gs) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (s0 + e >= a && s0 + e < end && gs + e < col_capacity) col_idx[gs + e] = st[s0 + e];
        }
      }
      wave_sync_lds();  // ... and the reads precede the next block's writes
      base += total_blk;
    }
  }
}

__global__ __launch_bounds__(64 * kFillWaves) void compact_fill_kernel(
    const uint32_t* __restrict__ mask, long long rows, int words, int T_k,
    const int32_t* __restrict__ counts, const long long* __restrict__ group_offsets,
    const long long* __restrict__ total, long long* __restrict__ row_ptr,
    int32_t* __restrict__ col_idx, long long col_capacity) {
  // a block's kept tiles per wave (up to 64 * 32), after up to 3 alignment slots
  __shared__ __attribute__((aligned(16))) int32_t stage[kFillWaves][64 * 32 + 4];
  const int wave = wave_uniform(threadIdx.x >> 6);
  const long long fill_groups = (rows + kFillWaves - 1) / kFillWaves;
  for (long long fg = blockIdx.x; fg < fill_groups; fg += gridDim.x) {
    const long long row = fg * kFillWaves + wave;
    if (row < rows)
      fill_row(mask, row, rows, words, T_k, counts, group_offsets, total, row_ptr, col_idx, col_capacity,
               stage[wave]);
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
  hipLaunchKernelGGL(compact_count_kernel, dim3(stride_blocks(groups, 1)), dim3(64 * kRowsPerGroup), 0, stream, mask,
                     rows, words, T_k, counts, gsum);
  hipLaunchKernelGGL(scan_groups_kernel, dim3(1), dim3(1024), 0, stream, gsum, groups, total);
  hipLaunchKernelGGL(compact_fill_kernel, dim3(stride_blocks(fill_groups, 1)), dim3(64 * kFillWaves), 0, stream, mask, rows,
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
