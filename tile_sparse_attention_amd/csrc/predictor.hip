// Tile-mask predictor from pooled queries and keys.
//
// The FG-Attn abstract ("FG-Attn: Leveraging Fine-Grained Sparse Attention in
// Video Diffusion Models", section Abstract) runs attention on an M x N tile
// keep-mask; this produces such a mask cheaply:
//   1. pool:    Qbar_i = mean of the valid rows of query tile i, Kbar_j = mean
//               of the keys of key tile j (fp32 sums of the input elements);
//   2. score:   s_ij = Qbar_i . Kbar_j for a block of query-tile rows, an fp32
//               matrix-core product (16x16x4 MFMA) staged through LDS;
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

template <typename E>
__global__ __launch_bounds__(256) void pool_tiles_kernel(const E* __restrict__ x, float* __restrict__ out,
                                                         long long total, int L, int d, int T,
                                                         int tile) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
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
  out[idx] = s / (float)(r1 - r0);
}

// scores[z][r][j] = Qbar[bh0+z][i0+r] . Kbar[bh0+z][j] for r < rows, j < T_k.
template <int D>
__global__ __launch_bounds__(256) void pooled_scores_kernel(const float* __restrict__ qbar,
                                                            const float* __restrict__ kbar,
                                                            float* __restrict__ scores, int T_q,
                                                            int T_k, int T_kp, int i0, int rows,
                                                            int R, int bh0) {
  constexpr int S = D + 4;  // +16 B row padding
  __shared__ __attribute__((aligned(16))) float qs[64 * S];
  __shared__ __attribute__((aligned(16))) float ks[64 * S];
  const int tid = threadIdx.x;
  const int bh = bh0 + blockIdx.z;
  const int rbase = 64 * blockIdx.y;  // row within the block of rows
  const int cbase = 64 * blockIdx.x;
  constexpr int CH = D / 4;           // float4 chunks per row
  // loads from clamped rows, out-of-range ones zeroed after: no branch
  // between them, so four iterations' loads are in flight together
#pragma unroll 4
  for (int e = tid; e < 64 * CH; e += 256) {
    const int rr = e / CH, c4 = e % CH;
    const int r = rbase + rr, j = cbase + rr;
    const int rc = r < rows ? r : rows - 1, jc = j < T_k ? j : T_k - 1;
    f32x4 a = *reinterpret_cast<const f32x4*>(qbar + ((size_t)bh * T_q + i0 + rc) * D + 4 * c4);
    f32x4 b = *reinterpret_cast<const f32x4*>(kbar + ((size_t)bh * T_k + jc) * D + 4 * c4);
    if (r >= rows) a = f32x4{0.f, 0.f, 0.f, 0.f};
    if (j >= T_k) b = f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(&qs[rr * S + 4 * c4]) = a;
    *reinterpret_cast<f32x4*>(&ks[rr * S + 4 * c4]) = b;
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  f32x4 acc[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) acc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int kk = 0; kk < D / 16; ++kk) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(&qs[(16 * wave + n) * S + 16 * kk + 4 * g]);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const f32x4 b = *reinterpret_cast<const f32x4*>(&ks[(16 * jb + n) * S + 16 * kk + 4 * g]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[jb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc[jb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    const int j = cbase + 16 * jb + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rbase + 16 * wave + 4 * g + i;
      if (r < rows && j < T_k) scores[((size_t)blockIdx.z * R + r) * T_kp + j] = acc[jb][i];
    }
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
  // Per-pass histogram in 16 copies, one per lane index mod 16, 257 ints
  // apart so the copies of a bin sit in different banks: score digits
  // crowd into a few bins (the top byte holds the sign and exponent), and
  // one shared copy would serialise a wave's atomics on them.
  constexpr int HC = 16, HS = 257;
  __shared__ int hist16[HC * HS];
  __shared__ int hist[256];
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

  // -- radix select of the k-th largest key, 8 bits at a time --
  uint32_t prefix = 0, pmask = 0;
  int kr = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int e = tid; e < HC * HS; e += 256) hist16[e] = 0;
    __syncthreads();
    int* hl = hist16 + (lane & (HC - 1)) * HS;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      const int j = tid + 256 * t;
      if (j >= T_k) break;
      const uint32_t key = key_at(t, j);
      if ((key & pmask) == prefix) atomicAdd(&hl[(key >> shift) & 255], 1);
    }
    __syncthreads();
    {
      int sum = 0;
#pragma unroll
      for (int c = 0; c < HC; ++c) sum += hist16[c * HS + tid];
      hist[tid] = sum;
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins 255-4l .. 252-4l (descending); inclusive scan over lanes
      int c[4], s = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) { c[q] = hist[255 - 4 * lane - q]; s += c[q]; }
      int inc = s;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
      }
      const int exc = inc - s;
      if (exc < kr && inc >= kr) {
        int cum = exc;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (cum + c[q] >= kr) {
            sh_prefix = prefix | ((uint32_t)(255 - 4 * lane - q) << shift);
            sh_kr = kr - cum;
            sh_eqn = c[q];  // after the last digit: the keys equal to the k-th largest
            break;
          }
          cum += c[q];
        }
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    kr = sh_kr;
    pmask |= 255u << shift;
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
  size_t qbar_bytes, kbar_bytes, score_bytes;
};

// Scores are materialised for G heads x R rows at a time, within a 512 MiB cap.
static PredictPlan predict_plan(const tsa_problem_t* p) {
  PredictPlan pl;
  pl.T_q = (p->L + p->M - 1) / p->M;
  pl.T_k = (p->L + p->N - 1) / p->N;
  pl.T_kp = (pl.T_k + 63) / 64 * 64;
  pl.words = (pl.T_k + 31) / 32;
  const size_t cap = (size_t)512 << 20;
  const size_t row_bytes = (size_t)pl.T_kp * sizeof(float);
  const size_t head_bytes = row_bytes * (size_t)pl.T_q;
  const int BH = p->B * p->H;
  if (head_bytes <= cap) {
    pl.R = pl.T_q;
    pl.G = (int)(cap / head_bytes);
    if (pl.G > BH) pl.G = BH;
    if (pl.G < 1) pl.G = 1;
  } else {
    pl.G = 1;
    long long r = (long long)(cap / row_bytes) / 64 * 64;
    if (r < 64) r = 64;
    pl.R = (int)(r < pl.T_q ? r : pl.T_q);
  }
  pl.qbar_bytes = ((size_t)BH * pl.T_q * p->d * sizeof(float) + 255) & ~(size_t)255;
  pl.kbar_bytes = ((size_t)BH * pl.T_k * p->d * sizeof(float) + 255) & ~(size_t)255;
  pl.score_bytes = (size_t)pl.G * pl.R * row_bytes;
  return pl;
}

size_t predict_workspace(const tsa_problem_t* p) {
  const PredictPlan pl = predict_plan(p);
  return pl.qbar_bytes + pl.kbar_bytes + pl.score_bytes;
}

hipError_t launch_predict_mask(const tsa_problem_t* p, const void* q, const void* k,
                               int sparsity_percent, uint32_t* mask_out, void* workspace,
                               hipStream_t stream) {
  const PredictPlan pl = predict_plan(p);
  char* ws = static_cast<char*>(workspace);
  float* qbar = reinterpret_cast<float*>(ws);
  float* kbar = reinterpret_cast<float*>(ws + pl.qbar_bytes);
  float* sc = reinterpret_cast<float*>(ws + pl.qbar_bytes + pl.kbar_bytes);
  const int BH = p->B * p->H;
  const long long nq = (long long)BH * pl.T_q * p->d;
  const long long nk = (long long)BH * pl.T_k * p->d;
  if (p->dtype == TSA_DTYPE_BF16) {
    hipLaunchKernelGGL(pool_tiles_kernel<bf16_t>, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0,
                       stream, static_cast<const bf16_t*>(q), qbar, nq, p->L, p->d, pl.T_q, p->M);
    hipLaunchKernelGGL(pool_tiles_kernel<bf16_t>, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0,
                       stream, static_cast<const bf16_t*>(k), kbar, nk, p->L, p->d, pl.T_k, p->N);
  } else {
    hipLaunchKernelGGL(pool_tiles_kernel<float>, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0,
                       stream, static_cast<const float*>(q), qbar, nq, p->L, p->d, pl.T_q, p->M);
    hipLaunchKernelGGL(pool_tiles_kernel<float>, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0,
                       stream, static_cast<const float*>(k), kbar, nk, p->L, p->d, pl.T_k, p->N);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int kk = pl.T_k - 1 - (int)(((long long)sparsity_percent * (pl.T_k - 1)) / 100);
  for (int bh0 = 0; bh0 < BH; bh0 += pl.G) {
    const int G = BH - bh0 < pl.G ? BH - bh0 : pl.G;
    for (int i0 = 0; i0 < pl.T_q; i0 += pl.R) {
      const int rows = pl.T_q - i0 < pl.R ? pl.T_q - i0 : pl.R;
      const dim3 grid((unsigned)(pl.T_kp / 64), (unsigned)((rows + 63) / 64), (unsigned)G);
      if (p->d == 128)
        hipLaunchKernelGGL(pooled_scores_kernel<128>, grid, dim3(256), 0, stream, qbar, kbar, sc,
                           pl.T_q, pl.T_k, pl.T_kp, i0, rows, pl.R, bh0);
      else
        hipLaunchKernelGGL(pooled_scores_kernel<64>, grid, dim3(256), 0, stream, qbar, kbar, sc,
                           pl.T_q, pl.T_k, pl.T_kp, i0, rows, pl.R, bh0);
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
