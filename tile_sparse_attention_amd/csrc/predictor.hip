// Tile-mask predictor from pooled queries and keys.
//
// The FG-Attn abstract ("FG-Attn: Leveraging Fine-Grained Sparse Attention in
// Video Diffusion Models", section Abstract) runs attention on an M x N tile
// keep-mask; this produces such a mask cheaply:
//   1. pool:    Qbar_i = mean of the valid rows of query tile i, Kbar_j = mean
//               of the keys of key tile j (fp32 sums of the input elements),
//               each stored as a bf16 high part and a bf16 low part;
//   2. score:   s_ij = Qbar_i . Kbar_j on the bf16 matrix cores with each fp32
//               operand split into two bf16 parts (three products per pair);
//   3. select:  per row, the k highest scores, equal scores going to the
//               smaller j, packed into the row's keep bits.
// k = T_k - 1 - floor(sparsity * (T_k - 1) / 100): with distinct scores these
// are the tiles strictly above the row's linearly interpolated percentile.
//
// Steps 2 and 3 run in one kernel and no score is ever stored: a work-group
// owns 64 query-tile rows and streams the head's pooled keys past them three
// times.
//   pass 1  mean mu and spread sigma of each row's scores (high parts only,
//           over an even quarter of the keys of rows longer than 2048 tiles);
//   pass 2  full scores counted into a per-row histogram over the window
//           [mu - a sigma', mu + b sigma'] (sigma' = sigma with a margin),
//           with a = sqrt(1/q - 1), b = sqrt(1/p - 1), p = k / T_k,
//           q = (T_k - k + 1) / T_k: by Cantelli's inequality the k-th largest
//           of any set of T_k values with that mean and spread lies in it;
//           scores above the window are counted apart;
//   pass 3  the same scores again: tiles above the bin that holds the k-th
//           largest are kept, and that bin's scores (a few dozen) are
//           collected with their j in LDS, where the ones to keep are picked
//           exactly (by score, then by smaller j).
// A row whose k-th largest falls outside its window, or whose bin holds more
// than kPredCap scores (many equal scores), is finished by a second kernel
// that recomputes the row's scores on the vector units and runs an exact
// radix select over them.
#include <cmath>

#include "tsa_device.h"
#include "tsa.h"

namespace tsa {

// out_hi/out_lo[bh][t][dd]: the fp32 mean of tile t's valid rows of x at
// column dd, split into a bf16 high part (round to nearest even) and a bf16
// low part (the rounded remainder), the operands of the split-precision
// score product below.  The first thread also clears *clear (the count of
// rows left to the exact fallback kernel), when given.
template <typename E>
__global__ __launch_bounds__(256) void pool_tiles_kernel(const E* __restrict__ x, bf16_t* __restrict__ out_hi,
                                                         bf16_t* __restrict__ out_lo, long long total, int L,
                                                         int d, int T, int tile, int* __restrict__ clear) {
  if (clear != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *clear = 0;
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

// Order-preserving 32-bit key of a float (larger float, larger key; -0 = +0).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kPredRows = 64;  // query-tile rows per work-group
constexpr int kPredCap = 64;   // scores of a row's threshold bin held in LDS

// Histogram bins of one row: 128 words, as 256 bins of 16-bit counts (rows of
// at most 65535 key tiles) or 128 bins of 32-bit counts (longer rows).
template <bool WIDE>
struct PredBins {
  static constexpr int NB = WIDE ? 128 : 256;
  __device__ static int word(int b) { return WIDE ? b : b >> 1; }
  __device__ static uint32_t inc(int b) { return WIDE ? 1u : 1u << ((b & 1) * 16); }
  __device__ static int count(uint32_t w, int b) { return WIDE ? (int)w : (int)((w >> ((b & 1) * 16)) & 0xffffu); }
};

// The work-group's 64 query-tile rows stay in LDS (hi and lo planes, rows
// 2d + 32 bytes apart so that the 16-byte operand reads of 16 rows hit
// distinct banks).  Each wave takes the 32-key blocks w, w + 4, ... of the
// head and streams their pooled keys from L2 straight into registers, one
// 32-key block ahead, as the B operands of 16x16x32 products against all 64
// rows: no key staging and no barrier per block.  Lane (g, n) of a 16-key
// half holds the scores of rows 16 rb + 4g + i (rb, i < 4) for key n.
template <int D, bool WIDE>
__global__ __launch_bounds__(256, 2) void predict_fused_kernel(
    const bf16_t* __restrict__ qhi, const bf16_t* __restrict__ qlo, const bf16_t* __restrict__ khi,
    const bf16_t* __restrict__ klo, uint32_t* __restrict__ mask, int* __restrict__ fb_list,
    int* __restrict__ fb_count, int T_q, int T_k, int words, int k, float wa, float wb, int blk0, int nblocks) {
  using Bn = PredBins<WIDE>;
  constexpr int R = kPredRows, NS = D / 32, RB = 2 * D, RS = RB + 32, NB = Bn::NB, CAP = kPredCap;
  __shared__ __attribute__((aligned(16))) uint8_t qs_h[R * RS];
  __shared__ __attribute__((aligned(16))) uint8_t qs_l[R * RS];
  // per row: its histogram (128 words), later its threshold-bin scores
  // (64 order keys, then their 64 j)
  __shared__ __attribute__((aligned(16))) uint32_t hs[R * 128];
  __shared__ float mom[4][R][3];  // per wave and row: shift, sum and sum of squares of deviations
  __shared__ float mcnt[4];       // keys each wave saw
  __shared__ int ok_sh[R];        // the row has a usable window
  __shared__ int ca_sh[R];        // scores above the window
  __shared__ int bs_sh[R];        // threshold bin, -1: row left to the fallback
  __shared__ int kr_sh[R];        // scores of the threshold bin to keep
  __shared__ int cn_sh[R];        // scores in the threshold bin
  __shared__ int cc_sh[R];        // scores collected so far in pass 3

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int rblocks = (T_q + R - 1) / R;
  const int lb = blk0 + xcd_major_block((int)blockIdx.x, nblocks);
  const int bh = lb / rblocks;
  const int i0 = (lb - bh * rblocks) * R;
  const int rows = T_q - i0 < R ? T_q - i0 : R;
  const size_t row0 = (size_t)bh * T_q + i0;  // first global row of the work-group

  if (k <= 0) {  // a single key tile: nothing lies strictly above the percentile
    for (int e = tid; e < rows * words; e += 256) mask[row0 * words + e] = 0u;
    return;
  }
  // the rows' pooled queries to LDS (rows past T_q as zeros), histograms cleared
  for (int e = tid; e < R * (RB / 16); e += 256) {
    const int r = e / (RB / 16), c = e - r * (RB / 16);
    u32x4 h = u32x4{0u, 0u, 0u, 0u}, l = h;
    if (r < rows) {
      h = *reinterpret_cast<const u32x4*>(qhi + (row0 + r) * D + 8 * c);
      l = *reinterpret_cast<const u32x4*>(qlo + (row0 + r) * D + 8 * c);
    }
    *reinterpret_cast<u32x4*>(qs_h + r * RS + 16 * c) = h;
    *reinterpret_cast<u32x4*>(qs_l + r * RS + 16 * c) = l;
  }
  for (int e = tid; e < R * 32; e += 256) reinterpret_cast<u32x4*>(hs)[e] = u32x4{0u, 0u, 0u, 0u};
  if (tid < R) {
    ca_sh[tid] = 0;
    cc_sh[tid] = 0;
  }
  __syncthreads();

  // this wave's 16-key blocks when the work-group takes every st-th 32-key
  // block: q -> keys 32 st (wave + 4 (q >> 1)) + 16 (q & 1) + n
  const int nsb = (T_k + 31) / 32;
  auto nblocks_at = [&](int st) {
    return st * wave < nsb ? 2 * ((nsb - st * wave + 4 * st - 1) / (4 * st)) : 0;
  };
  auto kbase = [&](int q, int st) { return 32 * st * (wave + 4 * (q >> 1)) + 16 * (q & 1); };
  const __amdgpu_buffer_rsrc_t rkh = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(khi + (size_t)bh * T_k * D), (short)0, T_k * RB, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rkl = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(klo + (size_t)bh * T_k * D), (short)0, T_k * RB, kBufferFlags);
  // slab sl of block q's B operands (keys past T_k read as zero: offsets
  // past the resource)
  auto load = [&](int q, int st, int sl, u32x4& kh, u32x4& kl, bool full) {
    const uint32_t o = (uint32_t)(kbase(q, st) + n) * RB + 16 * g + 64 * sl;
    kh = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rkh, o, 0, 0));
    if (full) kl = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rkl, o, 0, 0));
  };
  const lds_cptr pqh = to_lds(qs_h) + n * RS + 16 * g;
  const lds_cptr pql = to_lds(qs_l) + n * RS + 16 * g;
  // every block of the wave: its scores against the 64 rows, the two 16-key
  // blocks of a 32-key block together so that each query operand read from
  // LDS feeds both.  Each slab's registers are refilled with the next 32-key
  // block's slab as soon as its products are issued.
  auto run = [&](bool full, int st, auto&& body) {
    const int nq = nblocks_at(st);
    if (nq == 0) return;
    u32x4 h0[NS], l0[NS], h1[NS], l1[NS];
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      load(0, st, sl, h0[sl], l0[sl], full);
      load(1, st, sl, h1[sl], l1[sl], full);
    }
    for (int q = 0; q < nq; q += 2) {  // nq is even
      // the query operands are the same for every block: read them again
      // per block rather than holding all of them in registers
      const int z = opaque_zero();
      f32x4 a0[4], a1[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) a0[rb] = a1[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const u32x4 ah = lds_read16(pqh + z + 16 * rb * RS + 64 * sl);
          a0[rb] = mfma_bf16(ah, h0[sl], a0[rb]);
          a1[rb] = mfma_bf16(ah, h1[sl], a1[rb]);
          if (full) {
            const u32x4 al = lds_read16(pql + z + 16 * rb * RS + 64 * sl);
            a0[rb] = mfma_bf16(ah, l0[sl], a0[rb]);
            a1[rb] = mfma_bf16(ah, l1[sl], a1[rb]);
            a0[rb] = mfma_bf16(al, h0[sl], a0[rb]);
            a1[rb] = mfma_bf16(al, h1[sl], a1[rb]);
          }
        }
        if (q + 2 < nq) {
          load(q + 2, st, sl, h0[sl], l0[sl], full);
          load(q + 3, st, sl, h1[sl], l1[sl], full);
        }
      }
      body(kbase(q, st), q, a0);
      body(kbase(q + 1, st), q + 1, a1);
    }
  };

  // ---- pass 1: mean and spread of each row's scores (high parts only) over
  // every fourth 32-key block of rows longer than 2048 key tiles, a sample
  // spread evenly over the row (the moments only place the window: a row
  // whose k-th largest falls outside it goes to the fallback), per wave as
  // deviations from the wave's score of its first key ----
  {
    float c0[4][4], s1[4][4], s2[4][4], cnt = 0.f;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) c0[rb][i] = s1[rb][i] = s2[rb][i] = 0.f;
    run(false, nsb > 64 ? 4 : 1, [&](int kb, int q, const f32x4 (&acc)[4]) {
      if (q == 0) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) c0[rb][i] = __shfl(acc[rb][i], lane & 48);
      }
      const bool in = kb + n < T_k;
      cnt += in ? 1.f : 0.f;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float dv = in ? acc[rb][i] - c0[rb][i] : 0.f;
          s1[rb][i] += dv;
          s2[rb][i] = fmaf(dv, dv, s2[rb][i]);
        }
    });
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) cnt += __shfl_xor(cnt, m);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = s1[rb][i], b = s2[rb][i];
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) {
          a += __shfl_xor(a, m);
          b += __shfl_xor(b, m);
        }
        if (n == 0) {
          const int r = 16 * rb + 4 * g + i;
          mom[wave][r][0] = c0[rb][i];
          mom[wave][r][1] = a;
          mom[wave][r][2] = b;
        }
      }
    if (lane == 0) mcnt[wave] = cnt;
  }
  __syncthreads();
  // the rows' windows, the four waves' moments combined about wave 0's shift.
  // A score s is placed by x = (s - lo) inv, monotone in s: bin floor(x) for
  // 0 <= x < NB, above the window for x >= NB.  A row without a window gets
  // lo = +inf, inv = 0, so x is NaN and it is counted nowhere.
  float wlo[4][4], winv[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rb + 4 * g + i;
      const float c = mom[0][r][0];
      const float ns = mcnt[0] + mcnt[1] + mcnt[2] + mcnt[3];  // keys sampled
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float nw = mcnt[w], dc = mom[w][r][0] - c, sw = mom[w][r][1];
        a += sw + nw * dc;
        b += mom[w][r][2] + 2.f * dc * sw + nw * dc * dc;
      }
      const float md = a / ns;
      const float var = fmaxf(b / ns - md * md, 0.f);
      const float mu = c + md;
      const float sd = sqrtf(var);
      const float sdw = sd * 1.0625f + 1e-5f * fabsf(mu);
      const float lo = mu - wa * sdw, hi = mu + wb * sdw;
      const float inv = (float)NB / (hi - lo);
      const bool ok = r < rows && hi - lo > 0.f && __builtin_isfinite(inv) && __builtin_isfinite(lo) &&
                      __builtin_isfinite(hi);
      wlo[rb][i] = ok ? lo : __builtin_inff();
      winv[rb][i] = ok ? inv : 0.f;
      if (wave == 0 && n == 0) ok_sh[r] = ok ? 1 : 0;
    }

  // ---- pass 2: histogram of each row's scores in its window ----
  {
    int ca[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) ca[rb][i] = 0;
    run(true, 1, [&](int kb, int, const f32x4 (&acc)[4]) {
      const bool in = kb + n < T_k;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = (acc[rb][i] - wlo[rb][i]) * winv[rb][i];
          if (in && x >= (float)NB) {
            ++ca[rb][i];
          } else if (in && x >= 0.f) {
            const int b = (int)x;
            const int r = 16 * rb + 4 * g + i;
            atomicAdd(&hs[r * 128 + (Bn::word(b) ^ (r & 31))], Bn::inc(b));
          }
        }
    });
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int a = ca[rb][i];
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) a += __shfl_xor(a, m);
        if (n == 0 && a != 0) atomicAdd(&ca_sh[16 * rb + 4 * g + i], a);
      }
  }
  __syncthreads();
  // threshold bin of each row (wave w: rows 16w .. 16w + 15): lane l holds
  // the bins NB-1-PER l .. NB-PER-PER l (descending), scanned across the wave
  constexpr int PER = NB / 64;
  for (int rl = 0; rl < 16; ++rl) {
    const int r = 16 * wave + rl;
    if (r >= rows) break;
    const int need = ok_sh[r] ? k - ca_sh[r] : 0;
    int bs = -1, kr = 0, cn = 0;
    if (need > 0) {
      int cnt[PER], sum = 0;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int b = NB - 1 - PER * lane - q;
        cnt[q] = Bn::count(hs[r * 128 + (Bn::word(b) ^ (r & 31))], b);
        sum += cnt[q];
      }
      int inc = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
      }
      const uint64_t reach = __ballot(inc >= need);
      if (reach != 0ull) {  // else the k-th largest lies below the window
        const int L = __builtin_ctzll(reach);
        int cum = inc - sum, fb = 0, fk = 0, fc = 0;
        bool found = false;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          if (!found && cum + cnt[q] >= need) {
            found = true;
            fb = NB - 1 - PER * lane - q;
            fk = need - cum;
            fc = cnt[q];
          }
          cum += cnt[q];
        }
        bs = __shfl(fb, L);
        kr = __shfl(fk, L);
        cn = __shfl(fc, L);
        if (cn > CAP) bs = -1;
      }
    }
    if (lane == 0) {
      bs_sh[r] = bs;
      kr_sh[r] = kr;
      cn_sh[r] = cn;
      if (bs < 0) fb_list[atomicAdd(fb_count, 1)] = (int)(row0 + r);
    }
  }
  __syncthreads();  // every row's bin is known; the histograms are free

  // ---- pass 3: keep bits above the threshold bin; that bin's scores to LDS ----
  // With x as in pass 2, a score lies above the threshold bin b (or above the
  // window) iff x >= b + 1, and in it iff not that and x >= b.  Rows left to
  // the fallback keep nothing here (threshold +inf).
  float tk[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rb + 4 * g + i;
      const int bs = r < rows ? bs_sh[r] : -1;
      tk[rb][i] = bs >= 0 ? (float)(bs + 1) : __builtin_inff();
    }
  // lane l stores the word of row l: keys 32 sb .. 32 sb + 31 of its super-block
  const int srb = lane >> 4, sg = (lane >> 2) & 3, si = lane & 3;
  const bool sok = lane < rows && bs_sh[lane] >= 0;
  uint32_t* __restrict__ srow = mask + (row0 + lane) * (size_t)words;
  uint32_t word = 0u;
  run(true, 1, [&](int kb, int q, const f32x4 (&acc)[4]) {
    const bool in = kb + n < T_k;
    uint32_t half = 0u;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = acc[rb][i];
        const float x = (s - wlo[rb][i]) * winv[rb][i];
        const bool keep = in && x >= tk[rb][i];
        const uint64_t bal = __ballot(keep);
        if (rb == srb && i == si) half = (uint32_t)(bal >> (16 * sg)) & 0xffffu;
        if (in && !keep && x >= tk[rb][i] - 1.f) {
          const int r = 16 * rb + 4 * g + i;
          const int pos = atomicAdd(&cc_sh[r], 1);
          if (pos < CAP) {
            hs[r * 128 + pos] = order_key(s);
            hs[r * 128 + 64 + pos] = (uint32_t)(kb + n);
          }
        }
      }
    if ((q & 1) == 0) {
      word = half;
    } else {
      word |= half << 16;
      const int w = kb >> 5;
      if (sok && w < words) srow[w] = word;
    }
  });
  __builtin_amdgcn_s_waitcnt(0);  // this wave's word stores have landed
  __syncthreads();                // ... and every wave's, before the ORs below
  // ---- the threshold bin's scores: keep the kr best (larger key, then smaller j) ----
  for (int rl = 0; rl < 16; ++rl) {
    const int r = 16 * wave + rl;
    if (r >= rows) break;
    if (bs_sh[r] < 0) continue;
    const int cnum = cc_sh[r];
    if (cnum != cn_sh[r]) {  // not the count pass 2 found: leave the row to the fallback
      if (lane == 0) fb_list[atomicAdd(fb_count, 1)] = (int)(row0 + r);
      continue;
    }
    const int kr = kr_sh[r];
    const uint32_t key = lane < cnum ? hs[r * 128 + lane] : 0u;
    const uint32_t j = lane < cnum ? hs[r * 128 + 64 + lane] : 0u;
    int rank = 0;  // candidates before this one: larger key, or equal key and smaller j
    for (int c = 0; c < cnum; ++c) {
      const uint32_t k2 = (uint32_t)__builtin_amdgcn_readlane((int)key, c);
      const uint32_t j2 = (uint32_t)__builtin_amdgcn_readlane((int)j, c);
      rank += (k2 > key || (k2 == key && j2 < j)) ? 1 : 0;
    }
    if (lane < cnum && rank < kr) atomicOr(&mask[(row0 + r) * words + (j >> 5)], 1u << (j & 31));
  }
}

// Rows of at most this many key tiles are scored once into LDS by the
// fallback kernel; longer rows are scored again on every pass.
constexpr int kFallbackRowMax = 8192;

// Exact select for the rows the fused kernel left (fb_list[0 .. *fb_count)):
// one work-group per row computes the row's scores on the vector units
// (fp32 fused multiply-adds of the same three split products), once into
// LDS or, for long rows, whenever it needs them, finds the k-th largest by a radix select over order-preserving
// keys (digits of 12, 10 and 10 bits, LDS histograms), and writes the row's
// words in full: keys above it, then the first (by ascending j) of the keys
// equal to it until k are kept.
template <int D>
__global__ __launch_bounds__(256) void predict_rows_fallback_kernel(
    const bf16_t* __restrict__ qhi, const bf16_t* __restrict__ qlo, const bf16_t* __restrict__ khi,
    const bf16_t* __restrict__ klo, uint32_t* __restrict__ mask, const int* __restrict__ fb_list,
    const int* __restrict__ fb_count, int T_q, int T_k, int words, int k) {
  __shared__ float qh_s[D], ql_s[D];
  __shared__ float row_s[kFallbackRowMax];
  __shared__ int hbin[4096];
  __shared__ int wsum[4];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_kr, sh_eqn;
  __shared__ int sh_eq[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nrows = *fb_count;
  for (int idx = blockIdx.x; idx < nrows; idx += gridDim.x) {
    const int grow = fb_list[idx];
    const int bh = grow / T_q;
    uint32_t* out = mask + (size_t)grow * words;
    __syncthreads();  // the previous row's readers of the LDS arrays are done
    for (int dd = tid; dd < D; dd += 256) {
      qh_s[dd] = bf16_to_f32(qhi[(size_t)grow * D + dd]);
      ql_s[dd] = bf16_to_f32(qlo[(size_t)grow * D + dd]);
    }
    __syncthreads();
    const bf16_t* kh0 = khi + (size_t)bh * T_k * D;
    const bf16_t* kl0 = klo + (size_t)bh * T_k * D;
    auto score_at = [&](int j) -> float {
      const u32x4* ph = reinterpret_cast<const u32x4*>(kh0 + (size_t)j * D);
      const u32x4* pl = reinterpret_cast<const u32x4*>(kl0 + (size_t)j * D);
      float s = 0.f;
#pragma unroll 4
      for (int c = 0; c < D / 8; ++c) {
        const u32x4 h = ph[c], l = pl[c];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t wh = h[e >> 1], wlo = l[e >> 1];
          const float kh = __uint_as_float((e & 1) ? (wh & 0xffff0000u) : (wh << 16));
          const float kl = __uint_as_float((e & 1) ? (wlo & 0xffff0000u) : (wlo << 16));
          const float qh = qh_s[8 * c + e], ql = ql_s[8 * c + e];
          s = fmaf(qh, kh, s);
          s = fmaf(qh, kl, s);
          s = fmaf(ql, kh, s);
        }
      }
      return s;
    };
    const bool in_lds = T_k <= kFallbackRowMax;
    if (in_lds) {
      for (int j = tid; j < T_k; j += 256) row_s[j] = score_at(j);
      __syncthreads();
    }
    auto key_at = [&](int j) -> uint32_t { return order_key(in_lds ? row_s[j] : score_at(j)); };
    // radix select of the k-th largest key, digits of 12, 10 and 10 bits
    uint32_t prefix = 0, pmask = 0;
    int kr = k;
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 20 : pass == 1 ? 10 : 0;
      const int nb = pass == 0 ? 4096 : 1024;
      const uint32_t dmask = (uint32_t)nb - 1u;
      for (int e = tid; e < nb; e += 256) hbin[e] = 0;
      __syncthreads();
      for (int j = tid; j < T_k; j += 256) {
        const uint32_t key = key_at(j);
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
    // prefix = k-th largest key; keep key > prefix, and the first kr keys == prefix
    const bool all_eq = sh_eqn == kr;
    int eq_before = 0;  // equal keys at smaller j, across earlier rounds
    for (int base = 0; base < T_k; base += 256) {
      const int j = base + tid;
      const uint32_t key = j < T_k ? key_at(j) : 0u;
      const bool eq = j < T_k && key == prefix;
      bool keep;
      if (all_eq) {
        keep = j < T_k && key >= prefix;
      } else {
        const uint64_t eqb = __ballot(eq);
        if (lane == 0) sh_eq[wave] = __builtin_popcountll(eqb);
        __syncthreads();
        int before = eq_before;
        for (int w = 0; w < wave; ++w) before += sh_eq[w];
        const int rank = before + (int)prefix_count64(eqb);
        keep = j < T_k && (key > prefix || (eq && rank < kr));
        eq_before += sh_eq[0] + sh_eq[1] + sh_eq[2] + sh_eq[3];
        __syncthreads();
      }
      const uint64_t kb = __ballot(keep);
      const int w0 = (base >> 5) + 2 * wave;
      if (lane == 0 && w0 < words) out[w0] = (uint32_t)kb;
      if (lane == 1 && w0 + 1 < words) out[w0 + 1] = (uint32_t)(kb >> 32);
    }
  }
}

struct PredictPlan {
  int T_q, T_k, words;
  size_t q_plane_bytes, k_plane_bytes, list_bytes;
};

static PredictPlan predict_plan(const tsa_problem_t* p) {
  PredictPlan pl;
  pl.T_q = (p->L + p->M - 1) / p->M;
  pl.T_k = (p->L + p->N - 1) / p->N;
  pl.words = (pl.T_k + 31) / 32;
  const size_t BH = (size_t)p->B * p->H;
  // bf16 hi and lo planes of the pooled means
  pl.q_plane_bytes = (BH * pl.T_q * p->d * sizeof(bf16_t) + 255) & ~(size_t)255;
  pl.k_plane_bytes = (BH * pl.T_k * p->d * sizeof(bf16_t) + 255) & ~(size_t)255;
  // the fallback's row count (one 256-byte slot), then its row list
  pl.list_bytes = 256 + ((BH * pl.T_q * sizeof(int) + 255) & ~(size_t)255);
  return pl;
}

size_t predict_workspace(const tsa_problem_t* p) {
  const PredictPlan pl = predict_plan(p);
  return 2 * pl.q_plane_bytes + 2 * pl.k_plane_bytes + pl.list_bytes;
}

// Work-groups of the fallback kernel; each takes rows idx, idx + this, ...
constexpr int kFallbackGroups = 1024;

hipError_t launch_predict_mask(const tsa_problem_t* p, const void* q, const void* k,
                               int sparsity_percent, uint32_t* mask_out, void* workspace,
                               hipStream_t stream) {
  const PredictPlan pl = predict_plan(p);
  char* ws = static_cast<char*>(workspace);
  bf16_t* qhi = reinterpret_cast<bf16_t*>(ws);
  bf16_t* qlo = reinterpret_cast<bf16_t*>(ws + pl.q_plane_bytes);
  bf16_t* khi = reinterpret_cast<bf16_t*>(ws + 2 * pl.q_plane_bytes);
  bf16_t* klo = reinterpret_cast<bf16_t*>(ws + 2 * pl.q_plane_bytes + pl.k_plane_bytes);
  int* fb_count = reinterpret_cast<int*>(ws + 2 * pl.q_plane_bytes + 2 * pl.k_plane_bytes);
  int* fb_list = fb_count + 64;
  const long long BH = (long long)p->B * p->H;
  const long long nq = BH * pl.T_q * p->d;
  const long long nk = BH * pl.T_k * p->d;
  if (p->dtype == TSA_DTYPE_BF16) {
    hipLaunchKernelGGL(pool_tiles_kernel<bf16_t>, dim3(stride_blocks(nq, 256)), dim3(256), 0, stream,
                       static_cast<const bf16_t*>(q), qhi, qlo, nq, p->L, p->d, pl.T_q, p->M, fb_count);
    hipLaunchKernelGGL(pool_tiles_kernel<bf16_t>, dim3(stride_blocks(nk, 256)), dim3(256), 0, stream,
                       static_cast<const bf16_t*>(k), khi, klo, nk, p->L, p->d, pl.T_k, p->N, nullptr);
  } else {
    hipLaunchKernelGGL(pool_tiles_kernel<float>, dim3(stride_blocks(nq, 256)), dim3(256), 0, stream,
                       static_cast<const float*>(q), qhi, qlo, nq, p->L, p->d, pl.T_q, p->M, fb_count);
    hipLaunchKernelGGL(pool_tiles_kernel<float>, dim3(stride_blocks(nk, 256)), dim3(256), 0, stream,
                       static_cast<const float*>(k), khi, klo, nk, p->L, p->d, pl.T_k, p->N, nullptr);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int kk = pl.T_k - 1 - (int)(((long long)sparsity_percent * (pl.T_k - 1)) / 100);
  // Cantelli window multipliers: p = kk / T_k of the scores lie at or above
  // the k-th largest, q = (T_k - kk + 1) / T_k at or below it
  const double pf = (double)kk / pl.T_k, qf = (double)(pl.T_k - kk + 1) / pl.T_k;
  const float wa = (float)std::sqrt(qf < 1.0 ? 1.0 / qf - 1.0 : 0.0);
  const float wb = kk > 0 ? (float)std::sqrt(1.0 / pf - 1.0) : 0.f;
  const long long rblocks = (pl.T_q + kPredRows - 1) / kPredRows;
  const long long total = BH * rblocks;
  const bool wide = pl.T_k > 65535;
  for (long long b0 = 0; b0 < total; b0 += kMaxStrideBlocks) {
    const int nb = (int)(total - b0 < kMaxStrideBlocks ? total - b0 : kMaxStrideBlocks);
#define TSA_PRED_LAUNCH(D_, W_)                                                                            \
  hipLaunchKernelGGL((predict_fused_kernel<D_, W_>), dim3((unsigned)nb), dim3(256), 0, stream, qhi, qlo, khi, klo, \
                     mask_out, fb_list, fb_count, pl.T_q, pl.T_k, pl.words, kk, wa, wb, (int)b0, nb)
    if (p->d == 128) {
      if (wide) TSA_PRED_LAUNCH(128, true);
      else TSA_PRED_LAUNCH(128, false);
    } else {
      if (wide) TSA_PRED_LAUNCH(64, true);
      else TSA_PRED_LAUNCH(64, false);
    }
#undef TSA_PRED_LAUNCH
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (p->d == 128)
    hipLaunchKernelGGL(predict_rows_fallback_kernel<128>, dim3(kFallbackGroups), dim3(256), 0, stream, qhi, qlo,
                       khi, klo, mask_out, fb_list, fb_count, pl.T_q, pl.T_k, pl.words, kk);
  else
    hipLaunchKernelGGL(predict_rows_fallback_kernel<64>, dim3(kFallbackGroups), dim3(256), 0, stream, qhi, qlo,
                       khi, klo, mask_out, fb_list, fb_count, pl.T_q, pl.T_k, pl.words, kk);
  return hipGetLastError();
}

}  // namespace tsa
