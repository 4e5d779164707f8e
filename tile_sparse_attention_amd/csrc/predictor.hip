// Tile-mask predictor from pooled queries and keys.
//
// The FG-Attn abstract ("FG-Attn: Leveraging Fine-Grained Sparse Attention in
// Video Diffusion Models", section Abstract) runs attention on an M x N tile
// keep-mask; this produces such a mask cheaply:
//   1. pool:    Qbar_i = mean of the valid rows of query tile i, Kbar_j = mean
//               of the keys of key tile j (fp32 sums of the input elements),
//               each stored as a bf16 high part and a bf16 low part;
//   2. score:   s_ij = Qbar_i . Kbar_j for a block of query-tile rows, on the
//               bf16 matrix cores with each fp32 operand split into two bf16
//               parts (three products per pair), staged through LDS;
//   3. select:  per row (held in registers when it has at most 8192 key tiles), an
//               exact radix select of the k-th largest score on
//               order-preserving 32-bit keys, then keep everything above it
//               plus the first (by ascending j) of the scores equal to it, so
//               exactly k tiles are kept and ties go to the smaller j;
//               the decisions are packed 64 at a time with a wave ballot.
// k = T_k - 1 - floor(sparsity * (T_k - 1) / 100): with distinct scores these
// are the tiles strictly above the row's linearly interpolated percentile.
#include "tsa_device.h"
#include "tsa.h"

namespace tsa {

// out_hi/out_lo[bh][t][dd]: the fp32 mean of tile t's valid rows of x at
// column dd, split into a bf16 high part (round to nearest even) and a bf16
// low part (the rounded remainder), the operands of the split-precision
// score product below.
template <typename E>
__global__ __launch_bounds__(256) void pool_tiles_kernel(const E* __restrict__ x, bf16_t* __restrict__ out_hi,
                                                         bf16_t* __restrict__ out_lo, long long total, int L,
                                                         int d, int T, int tile) {
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (long long)gridDim.x * 256) {
    const int dd = (int)(idx % d);
    const long long bt = idx / d;
    const int t = (int)(bt % T);
    const long long bh = bt / T;
    const int r0 = t * tile;
    const int r1 = r0 + tile < L ? r0 + tile : L;
    const E* src = x + ((size_t)bh * L + r0) * d + dd;
    float s = 0.f;
#pragma unroll 8
    for (int r = r0; r < r1; ++r, src += d) {
      if constexpr (sizeof(E) == 2) s += bf16_to_f32(*reinterpret_cast<const bf16_t*>(src));
      else s += *src;
    }
    const float mean = s / (float)(r1 - r0);
    const __bf16 hi = (__bf16)mean;
    out_hi[idx] = __builtin_bit_cast(bf16_t, hi);
    out_lo[idx] = __builtin_bit_cast(bf16_t, (__bf16)(mean - (float)hi));
  }
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// scores[z][r][j] = Qbar[bh0+z][i0+r] . Kbar[bh0+z][j] for r < rows, j < T_k.
// Each fp32 mean x is held as x = hi + lo with hi, lo bf16, and a product as
// hi_q hi_k + hi_q lo_k + lo_q hi_k on the bf16 matrix cores (16x16x32, fp32
// accumulation): the dropped lo_q lo_k term and the rounding of lo leave a
// relative error near 2^-16 per term, against 2^-24 for fp32 products, at
// the bf16 rate instead of the fp32 matrix-core rate.
// A work-group owns 128 query-tile rows (wave w: rows 32w..32w+31, held as
// register operands) and a run of 128-wide key-tile blocks, which stream
// through two LDS buffers (hi and lo planes, rows 288 bytes apart: the
// 16-byte operand reads of 16 rows are free of bank conflicts) filled by
// direct global-to-LDS loads one block ahead.
constexpr int kScoreTile = 128;

template <int D>
struct ScoreGemm {
  static constexpr int TB = kScoreTile;
  static constexpr int RB = D * 2;                       // bf16 row bytes
  static constexpr int RS = RB + 32;                     // LDS row stride
  static constexpr int NI_T = (TB * RS + 1023) / 1024;   // 1-KB loads per plane tile
  static constexpr int NS = D / 32;                      // 32-wide d slabs
  struct Buf {
    __attribute__((aligned(16))) uint8_t hi[NI_T * 1024];
    __attribute__((aligned(16))) uint8_t lo[NI_T * 1024];
  };
};

template <int D>
__global__ __launch_bounds__(256) void pooled_scores_kernel(const bf16_t* __restrict__ qhi,
                                                            const bf16_t* __restrict__ qlo,
                                                            const bf16_t* __restrict__ khi,
                                                            const bf16_t* __restrict__ klo,
                                                            float* __restrict__ scores, int T_q, int T_k,
                                                            int T_kp, int i0, int rows, int R, int bh0,
                                                            int blocks_per_wg) {
  using G = ScoreGemm<D>;
  constexpr int TB = G::TB;
  __shared__ __attribute__((aligned(16))) typename G::Buf b0;
  __shared__ __attribute__((aligned(16))) typename G::Buf b1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int bh = bh0 + blockIdx.z;
  const int rbase = TB * blockIdx.y;
  const int nblk = T_kp / TB;
  const int t0 = blockIdx.x * blocks_per_wg;
  const int t1 = t0 + blocks_per_wg < nblk ? t0 + blocks_per_wg : nblk;
  if (t0 >= t1) return;
  // this wave's query operands: lane (g, n) holds row n of each 16-row
  // block, d = 32 sl + 8g .. +7 of each slab
  u32x4 ah[2][G::NS], al[2][G::NS];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = rbase + 32 * wave + 16 * rb + n;
    const size_t row = (size_t)bh * T_q + i0 + (r < rows ? r : rows - 1);
#pragma unroll
    for (int sl = 0; sl < G::NS; ++sl) {
      ah[rb][sl] = *reinterpret_cast<const u32x4*>(qhi + row * D + 32 * sl + 8 * g);
      al[rb][sl] = *reinterpret_cast<const u32x4*>(qlo + row * D + 32 * sl + 8 * g);
      if (r >= rows) ah[rb][sl] = al[rb][sl] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  // this wave's share of the loads of key block t into buffer bf: plane
  // rows of keys past T_k read as zero (out of the buffer's range), as do
  // the padding bytes of each LDS row
  auto issue = [&](int t, typename G::Buf& bf) {
    const int kb = t * TB;
    const int nrows = T_k - kb < TB ? T_k - kb : TB;
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(khi + ((size_t)bh * T_k + kb) * D), (short)0, nrows * G::RB, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(klo + ((size_t)bh * T_k + kb) * D), (short)0, nrows * G::RB, kBufferFlags);
    for (int I = wave; I < G::NI_T; I += 4) {
      const int pos = I * 1024 + 16 * lane;
      const int row = pos / G::RS, cb = pos - row * G::RS;
      const uint32_t off = row < TB && cb < G::RB ? (uint32_t)(row * G::RB + cb) : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (__attribute__((address_space(3))) void*)(bf.hi + I * 1024),
                                               16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (__attribute__((address_space(3))) void*)(bf.lo + I * 1024),
                                               16, off, 0, 0, 0);
    }
  };
  auto compute = [&](int t, const typename G::Buf& bf) {
    f32x4 acc[2][TB / 16];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int jb = 0; jb < TB / 16; ++jb) acc[rb][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const lds_cptr ph = to_lds(bf.hi) + n * G::RS + 16 * g;
    const lds_cptr pl = to_lds(bf.lo) + n * G::RS + 16 * g;
#pragma unroll
    for (int sl = 0; sl < G::NS; ++sl) {
#pragma unroll
      for (int jb = 0; jb < TB / 16; ++jb) {
        const u32x4 bh_ = lds_read16(ph + 16 * jb * G::RS + 64 * sl);
        const u32x4 bl_ = lds_read16(pl + 16 * jb * G::RS + 64 * sl);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          acc[rb][jb] = mfma_bf16(ah[rb][sl], bh_, acc[rb][jb]);
          acc[rb][jb] = mfma_bf16(ah[rb][sl], bl_, acc[rb][jb]);
          acc[rb][jb] = mfma_bf16(al[rb][sl], bh_, acc[rb][jb]);
        }
      }
    }
    // D[m][c] of block (rb, jb): lane (g, n) holds rows 4g..4g+3, column n
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int jb = 0; jb < TB / 16; ++jb) {
        const int j = t * TB + 16 * jb + n;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rbase + 32 * wave + 16 * rb + 4 * g + i;
          if (r < rows && j < T_k) scores[((size_t)blockIdx.z * R + r) * T_kp + j] = acc[rb][jb][i];
        }
      }
  };
  issue(t0, b0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // two blocks per iteration, so that each buffer is named statically
  for (int t = t0; t < t1; t += 2) {
    // buffer 1 was last read in the previous iteration, which every wave has left
    if (t + 1 < t1) issue(t + 1, b1);
    compute(t, b0);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of block t+1 have landed
    __syncthreads();                // ... and every other wave's; buffer 0 is free
    if (t + 1 >= t1) break;
    if (t + 2 < t1) issue(t + 2, b0);
    compute(t + 1, b1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Rows of up to this many key tiles are held in registers while they are
// selected (32 keys per thread: thread t owns tiles t, t + 256, ...); longer
// rows are read from the score block on every pass.
constexpr int kSelectRowMax = 8192;

template <bool IN_REG>
__global__ __launch_bounds__(256) void select_pack_kernel(const float* __restrict__ scores,
                                                          uint32_t* __restrict__ mask, int T_q,
                                                          int T_k, int T_kp, int words, int i0,
                                                          int rows, int R, int bh0, int k) {
  // Histogram of one digit (4096 bins for the first, 1024 for the others),
  // wave totals of its scan, and the pass's result.
  __shared__ int hbin[4096];
  __shared__ int wsum[4];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_kr, sh_eqn;
  __shared__ int sh_eq[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int z = blockIdx.x / rows, il = blockIdx.x % rows;
  const float* srow = scores + ((size_t)z * R + il) * T_kp;
  uint32_t* out = mask + ((size_t)(bh0 + z) * T_q + i0 + il) * words;
  if (k <= 0) {  // a single key tile: nothing lies strictly above the percentile
    for (int w = tid; w < words; w += 256) out[w] = 0u;
    return;
  }
  // the thread's keys, read from the score block once (every load issued
  // before the first is waited for); every later access of the thread is to
  // one of its own tiles t + 256 i
  constexpr int NPT = IN_REG ? kSelectRowMax / 256 : 1;
  uint32_t rk[NPT];
  if constexpr (IN_REG) {
#pragma unroll
    for (int t = 0; t < NPT; ++t) {
      const int j = tid + 256 * t;
      rk[t] = order_key(j < T_k ? srow[j] : 0.f);
    }
  }
  // key of tile j = tid + 256 * t
  auto key_at = [&](int t, int j) -> uint32_t {
    if constexpr (IN_REG) return rk[t];
    else return order_key(srow[j]);
  };
  constexpr int TMAX = IN_REG ? NPT : 0x7fffffff;  // bound of t (the real bound is j < T_k)

  // -- radix select of the k-th largest key: digits of 12, 10 and 10 bits.
  // The first digit (sign, exponent and three mantissa bits) spreads scores
  // over many bins; later digits count only the keys under the prefix found
  // so far, a few dozen at most. --
  uint32_t prefix = 0, pmask = 0;
  int kr = k;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : pass == 1 ? 10 : 0;
    const int nb = pass == 0 ? 4096 : 1024;
    const uint32_t dmask = (uint32_t)nb - 1u;
    for (int e = tid; e < nb; e += 256) hbin[e] = 0;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      const int j = tid + 256 * t;
      if (j >= T_k) break;
      const uint32_t key = key_at(t, j);
      if ((key & pmask) == prefix) atomicAdd(&hbin[(key >> shift) & dmask], 1);
    }
    __syncthreads();
    // thread t owns the digits nb-1-t*per .. nb-per-t*per (descending)
    const int per = nb >> 8;
    int s = 0;
    for (int q = 0; q < per; ++q) s += hbin[nb - 1 - tid * per - q];
    int inc = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(inc, off);
      if (lane >= off) inc += y;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    for (int w = 0; w < wave; ++w) inc += wsum[w];
    const int exc = inc - s;
    if (exc < kr && inc >= kr) {
      int cum = exc;
      for (int q = 0; q < per; ++q) {
        const int dgt = nb - 1 - tid * per - q;
        const int c = hbin[dgt];
        if (cum + c >= kr) {
          sh_prefix = prefix | ((uint32_t)dgt << shift);
          sh_kr = kr - cum;
          sh_eqn = c;  // after the last digit: the keys equal to the k-th largest
          break;
        }
        cum += c;
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    kr = sh_kr;
    pmask |= dmask << shift;
    __syncthreads();
  }
  // prefix = k-th largest key; keep key > prefix, and the first kr keys == prefix.
  if (sh_eqn == kr) {
    // every key equal to the k-th largest is kept (the usual case: no ties),
    // so each wave packs 64-key runs on its own, with no ranks to count
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      const int base = 64 * wave + 256 * t, j = base + lane;
      if (base >= T_k) break;
      const uint64_t kb = __ballot(j < T_k && key_at(t, j) >= prefix);
      const int w0 = base >> 5;
      if (lane == 0) out[w0] = (uint32_t)kb;
      if (lane == 1 && w0 + 1 < words) out[w0 + 1] = (uint32_t)(kb >> 32);
    }
    return;
  }
  int eq_before = 0;  // equal keys at smaller j, across earlier rounds
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    const int base = 256 * t, j = base + tid;
    if (base >= T_k) break;
    const uint32_t key = j < T_k ? key_at(t, j) : 0u;
    const bool eq = j < T_k && key == prefix;
    const uint64_t eqb = __ballot(eq);
    if (lane == 0) sh_eq[wave] = __builtin_popcountll(eqb);
    __syncthreads();
    int before = eq_before;
    for (int w = 0; w < wave; ++w) before += sh_eq[w];
    const int rank = before + (int)prefix_count64(eqb);
    const bool keep = j < T_k && (key > prefix || (eq && rank < kr));
    const uint64_t kb = __ballot(keep);
    const int w0 = (base >> 5) + 2 * wave;
    if (lane == 0 && w0 < words) out[w0] = (uint32_t)kb;
    if (lane == 1 && w0 + 1 < words) out[w0 + 1] = (uint32_t)(kb >> 32);
    eq_before += sh_eq[0] + sh_eq[1] + sh_eq[2] + sh_eq[3];
    __syncthreads();
  }
}

struct PredictPlan {
  int T_q, T_k, T_kp, words, R, G;
  size_t q_plane_bytes, k_plane_bytes, score_bytes;
};

// Scores are materialised for G heads x R rows at a time, within a 224 MiB
// cap: small enough that a block written by the score kernel is still in the
// chip's 256 MB memory-side cache when the select kernel reads it.
static PredictPlan predict_plan(const tsa_problem_t* p) {
  PredictPlan pl;
  pl.T_q = (p->L + p->M - 1) / p->M;
  pl.T_k = (p->L + p->N - 1) / p->N;
  pl.T_kp = (pl.T_k + kScoreTile - 1) / kScoreTile * kScoreTile;
  pl.words = (pl.T_k + 31) / 32;
  const size_t cap = (size_t)224 << 20;
  const size_t row_bytes = (size_t)pl.T_kp * sizeof(float);
  const size_t head_bytes = row_bytes * (size_t)pl.T_q;
  const int BH = p->B * p->H;
  if (head_bytes <= cap) {
    pl.R = pl.T_q;
    pl.G = (int)(cap / head_bytes);
    if (pl.G > BH) pl.G = BH;
    if (pl.G > 65535) pl.G = 65535;  // the score grid's third dimension
    if (pl.G < 1) pl.G = 1;
  } else {
    pl.G = 1;
    long long r = (long long)(cap / row_bytes) / kScoreTile * kScoreTile;
    if (r < kScoreTile) r = kScoreTile;
    pl.R = (int)(r < pl.T_q ? r : pl.T_q);
  }
  // bf16 hi and lo planes of the pooled means
  pl.q_plane_bytes = ((size_t)BH * pl.T_q * p->d * sizeof(bf16_t) + 255) & ~(size_t)255;
  pl.k_plane_bytes = ((size_t)BH * pl.T_k * p->d * sizeof(bf16_t) + 255) & ~(size_t)255;
  pl.score_bytes = (size_t)pl.G * pl.R * row_bytes;
  return pl;
}

size_t predict_workspace(const tsa_problem_t* p) {
  const PredictPlan pl = predict_plan(p);
  return 2 * pl.q_plane_bytes + 2 * pl.k_plane_bytes + pl.score_bytes;
}

hipError_t launch_predict_mask(const tsa_problem_t* p, const void* q, const void* k,
                               int sparsity_percent, uint32_t* mask_out, void* workspace,
                               hipStream_t stream) {
  const PredictPlan pl = predict_plan(p);
  char* ws = static_cast<char*>(workspace);
  bf16_t* qhi = reinterpret_cast<bf16_t*>(ws);
  bf16_t* qlo = reinterpret_cast<bf16_t*>(ws + pl.q_plane_bytes);
  bf16_t* khi = reinterpret_cast<bf16_t*>(ws + 2 * pl.q_plane_bytes);
  bf16_t* klo = reinterpret_cast<bf16_t*>(ws + 2 * pl.q_plane_bytes + pl.k_plane_bytes);
  float* sc = reinterpret_cast<float*>(ws + 2 * pl.q_plane_bytes + 2 * pl.k_plane_bytes);
  const int BH = p->B * p->H;
  const long long nq = (long long)BH * pl.T_q * p->d;
  const long long nk = (long long)BH * pl.T_k * p->d;
  if (p->dtype == TSA_DTYPE_BF16) {
    hipLaunchKernelGGL(pool_tiles_kernel<bf16_t>, dim3(stride_blocks(nq, 256)), dim3(256), 0, stream,
                       static_cast<const bf16_t*>(q), qhi, qlo, nq, p->L, p->d, pl.T_q, p->M);
    hipLaunchKernelGGL(pool_tiles_kernel<bf16_t>, dim3(stride_blocks(nk, 256)), dim3(256), 0, stream,
                       static_cast<const bf16_t*>(k), khi, klo, nk, p->L, p->d, pl.T_k, p->N);
  } else {
    hipLaunchKernelGGL(pool_tiles_kernel<float>, dim3(stride_blocks(nq, 256)), dim3(256), 0, stream,
                       static_cast<const float*>(q), qhi, qlo, nq, p->L, p->d, pl.T_q, p->M);
    hipLaunchKernelGGL(pool_tiles_kernel<float>, dim3(stride_blocks(nk, 256)), dim3(256), 0, stream,
                       static_cast<const float*>(k), khi, klo, nk, p->L, p->d, pl.T_k, p->N);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int kk = pl.T_k - 1 - (int)(((long long)sparsity_percent * (pl.T_k - 1)) / 100);
  const int nblk = pl.T_kp / kScoreTile;
  for (int bh0 = 0; bh0 < BH; bh0 += pl.G) {
    const int G = BH - bh0 < pl.G ? BH - bh0 : pl.G;
    for (int i0 = 0; i0 < pl.T_q; i0 += pl.R) {
      const int rows = pl.T_q - i0 < pl.R ? pl.T_q - i0 : pl.R;
      // key blocks split over work-groups so that one round of them (one per
      // compute unit: the two LDS buffers take most of its LDS) covers the
      // chip: each work-group streams its run of blocks past resident rows
      const int rblocks = (rows + kScoreTile - 1) / kScoreTile;
      int splits = 256 / (rblocks * G);
      if (splits < 1) splits = 1;
      if (splits > nblk) splits = nblk;
      const int per = (nblk + splits - 1) / splits;
      splits = (nblk + per - 1) / per;
      const dim3 grid((unsigned)splits, (unsigned)rblocks, (unsigned)G);
      if (p->d == 128)
        hipLaunchKernelGGL(pooled_scores_kernel<128>, grid, dim3(256), 0, stream, qhi, qlo, khi, klo, sc, pl.T_q,
                           pl.T_k, pl.T_kp, i0, rows, pl.R, bh0, per);
      else
        hipLaunchKernelGGL(pooled_scores_kernel<64>, grid, dim3(256), 0, stream, qhi, qlo, khi, klo, sc, pl.T_q,
                           pl.T_k, pl.T_kp, i0, rows, pl.R, bh0, per);
      if (pl.T_k <= kSelectRowMax)  // rows held in registers
        hipLaunchKernelGGL(select_pack_kernel<true>, dim3((unsigned)(G * rows)), dim3(256), 0, stream, sc,
                           mask_out, pl.T_q, pl.T_k, pl.T_kp, pl.words, i0, rows, pl.R, bh0, kk);
      else
        hipLaunchKernelGGL(select_pack_kernel<false>, dim3((unsigned)(G * rows)), dim3(256), 0, stream, sc,
                           mask_out, pl.T_q, pl.T_k, pl.T_kp, pl.words, i0, rows, pl.R, bh0, kk);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
  }
  return hipSuccess;
}

}  // namespace tsa
