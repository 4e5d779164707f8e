// Tile-sparse attention forward kernel (gfx950, wave64, MFMA).
//
// Operation: FG-Attn ("FG-Attn: Leveraging Fine-Grained Sparse Attention in
// Video Diffusion Models", section Abstract) skips the query-key dot products
// of every M x N tile whose keep bit is 0 and leaves those scores out of the
// softmax.  O = softmax(scale * Q K^T restricted to kept tiles) V.
//
// Work decomposition
//   * A work-group owns 16*W consecutive query rows of one (b, h); each wave
//     owns 16 of them (one 16-row slice of a mask row, since M is a multiple
//     of 16).
//   * Keys are streamed in chunks of KC keys.  The work-group stages each
//     chunk once in LDS (K as rows, V transposed to [d][key]) with
//     double-buffered, coalesced 16-byte global loads; every wave then reuses
//     it.  K/V are read from HBM/L2 once per work-group instead of once per
//     query tile.
//   * Per chunk each wave compacts its own mask bits into the list of kept
//     key tiles (wave prefix count of the bitmap, the same routine the
//     compaction kernel uses) and packs the kept keys densely into 16-key
//     "slots".  Matrix-core work is spent only on kept keys: a skipped tile
//     costs nothing beyond its mask bit, and kept tiles of any width N share
//     MFMA blocks instead of padding each tile to 16 keys.
//   * Scores are formed transposed, S^T = K Q^T (A = gathered K rows from LDS,
//     B = the wave's Q fragment held in registers), so each lane owns one
//     query column; the online softmax (running max m and sum l, base-2
//     exponent with scale*log2(e) folded in) is lane-local apart from a
//     4-lane-group max.  The S^T accumulator layout is directly the B operand
//     of O^T += V^T P^T, so probabilities never leave registers.
//   * Normalisation O = O / l (0 for a row with nothing kept) and the store
//     happen once at the end.
#pragma once

#include "tsa_device.h"

namespace tsa {

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const uint32_t* mask;
  void* o;
  float* lse;
  int H, L, M, T_q, T_k, words;
  int n_qblocks;
  float scale_log2;  // scale * log2(e)
};

template <typename T> struct ElemTraits;
template <> struct ElemTraits<float> { static constexpr int VEC = 4; };
template <> struct ElemTraits<bf16_t> { static constexpr int VEC = 8; };

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

template <typename T, int D, int N, int KC, int W>
struct AttnCfg {
  static constexpr int VEC = ElemTraits<T>::VEC;   // elements per 16 bytes
  static constexpr int SLAB = 4 * VEC;             // d covered by one 16-byte read per lane group
  static constexpr int NSLAB = D / SLAB;
  static constexpr int NDB = D / 16;               // 16-wide d blocks of O^T
  static constexpr int KSTR = D + VEC;             // K row stride in LDS (+16 B against bank conflicts)
  static constexpr int VSTR = KC + VEC;            // V^T row stride in LDS (+16 B)
  static constexpr int NT = 64 * W;
  static constexpr int CPR = D / VEC;              // 16-byte chunks per K/V row
  static constexpr int K_ITEMS = KC * CPR;
  static constexpr int V_ITEMS = (KC / 4) * CPR;   // groups of 4 rows x 16 bytes
  static constexpr int K_PER_T = (K_ITEMS + NT - 1) / NT;
  static constexpr int V_PER_T = (V_ITEMS + NT - 1) / NT;
  static constexpr int TPC = KC / N;               // key tiles per chunk
  static constexpr int WINT = TPC < 64 ? TPC : 64; // tiles per compaction window
  static constexpr int NWIN = TPC / WINT;
  static constexpr int LOG2N = ilog2(N);
  static constexpr int PASS_SB = 4;                // 16-slot sub-blocks per softmax pass
  static_assert(D % SLAB == 0 && D % 16 == 0, "head dim");
  static_assert(KC % N == 0 && KC % 64 == 0 && TPC <= 256, "chunk");
  static_assert((1 << LOG2N) == N, "N must be a power of two");
};

template <typename T> struct Mma;

template <> struct Mma<bf16_t> {
  // 16x16x32 bf16 -> fp32: one call consumes 8 k-values per lane.
  static __device__ __forceinline__ f32x4 mac8(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  // Four 16x16x4 fp32 steps, k-element e of each lane in step e.
  static __device__ __forceinline__ f32x4 mac4(u32x4 a, u32x4 b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), c, 0, 0,
                                               0);
    return c;
  }
};

template <typename T, int D, int N, int KC, int W>
__global__ __launch_bounds__(64 * W) void attn_fwd_kernel(AttnParams p) {
  using C = AttnCfg<T, D, N, KC, W>;
  constexpr int VEC = C::VEC;

  __shared__ __attribute__((aligned(16))) T k_lds[2][KC * C::KSTR];
  __shared__ __attribute__((aligned(16))) T vt_lds[2][D * C::VSTR];
  __shared__ uint8_t tlist[W][C::TPC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int wave = wave_uniform(tid >> 6);

  const int bh = blockIdx.x / p.n_qblocks;
  const int qb = blockIdx.x - bh * p.n_qblocks;
  const int L = p.L;
  const size_t head_off = (size_t)bh * (size_t)L * D;
  const T* __restrict__ qg = reinterpret_cast<const T*>(p.q) + head_off;
  const T* __restrict__ kg = reinterpret_cast<const T*>(p.k) + head_off;
  const T* __restrict__ vg = reinterpret_cast<const T*>(p.v) + head_off;

  const int row0 = qb * (16 * W) + 16 * wave;  // first query row of this wave
  const bool wave_active = row0 < L;
  const int mrow = row0 / p.M;
  const uint32_t* __restrict__ mask_row =
      p.mask + ((size_t)bh * p.T_q + (size_t)(wave_active ? mrow : 0)) * p.words;

  // ---- Q fragment: lane (g, n) holds Q[row0+n][SLAB*s + VEC*g .. +VEC) ----
  u32x4 qf[C::NSLAB];
  {
    const int r = row0 + n;
#pragma unroll
    for (int s = 0; s < C::NSLAB; ++s) {
      if (r < L)
        qf[s] = *reinterpret_cast<const u32x4*>(qg + (size_t)r * D + C::SLAB * s + VEC * g);
      else
        qf[s] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  f32x4 oacc[C::NDB];
#pragma unroll
  for (int j = 0; j < C::NDB; ++j) oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of scaled (log2-domain) scores of query n
  float l_run = 0.f;        // this lane group's share of the running sum

  // ---- chunk staging: global -> registers -> LDS ----
  u32x4 kreg[C::K_PER_T];
  u32x4 vreg[C::V_PER_T][4];

  auto load_chunk = [&](int c) {
    const int kbase = c * KC;
#pragma unroll
    for (int u = 0; u < C::K_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      if (C::K_ITEMS % C::NT == 0 || idx < C::K_ITEMS) {
        const int row = idx / C::CPR, ch = idx % C::CPR;
        const int key = kbase + row;
        kreg[u] = key < L ? *reinterpret_cast<const u32x4*>(kg + (size_t)key * D + ch * VEC)
                          : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      if (C::V_ITEMS % C::NT == 0 || idx < C::V_ITEMS) {
        const int rg = idx / C::CPR, ch = idx % C::CPR;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kbase + 4 * rg + r;
          vreg[u][r] = key < L ? *reinterpret_cast<const u32x4*>(vg + (size_t)key * D + ch * VEC)
                               : u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int u = 0; u < C::K_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      if (C::K_ITEMS % C::NT == 0 || idx < C::K_ITEMS) {
        const int row = idx / C::CPR, ch = idx % C::CPR;
        *reinterpret_cast<u32x4*>(&k_lds[buf][row * C::KSTR + ch * VEC]) = kreg[u];
      }
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      if (C::V_ITEMS % C::NT == 0 || idx < C::V_ITEMS) {
        const int rg = idx / C::CPR, ch = idx % C::CPR;
        T* dst = &vt_lds[buf][(ch * VEC) * C::VSTR + 4 * rg];
        const u32x4 r0 = vreg[u][0], r1 = vreg[u][1], r2 = vreg[u][2], r3 = vreg[u][3];
        if constexpr (sizeof(T) == 2) {
          // word w of a row holds d = 2w (low half) and 2w+1 (high half)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const u32x2 lo = {(r0[w] & 0xffffu) | (r1[w] << 16), (r2[w] & 0xffffu) | (r3[w] << 16)};
            const u32x2 hi = {(r0[w] >> 16) | (r1[w] & 0xffff0000u),
                              (r2[w] >> 16) | (r3[w] & 0xffff0000u)};
            *reinterpret_cast<u32x2*>(dst + (2 * w) * C::VSTR) = lo;
            *reinterpret_cast<u32x2*>(dst + (2 * w + 1) * C::VSTR) = hi;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            *reinterpret_cast<u32x4*>(dst + e * C::VSTR) = u32x4{r0[e], r1[e], r2[e], r3[e]};
        }
      }
    }
  };

  // key offset (within the chunk) of packed slot s, given this wave's tile list
  uint8_t* tl = tlist[wave];
  auto slot_key = [&](int s) -> int {
    if constexpr (N == 1) return (int)tl[s];
    else return ((int)tl[s >> C::LOG2N] << C::LOG2N) | (s & (N - 1));
  };

  // Four consecutive slots s0..s0+3 of V^T row `vrow` (all valid slots or
  // all dummies when N >= 4; dummies read key 0 and are multiplied by p = 0).
  auto vt_quad = [&](const T* vrow, int s0, int nslots) -> u32x4 {
    if constexpr (N >= 4) {
      const int key = s0 < nslots ? slot_key(s0) : 0;
      if constexpr (sizeof(T) == 2) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(vrow + key);
        return u32x4{x[0], x[1], 0u, 0u};
      } else {
        return *reinterpret_cast<const u32x4*>(vrow + key);
      }
    } else if constexpr (N == 2) {
      const int k0 = s0 < nslots ? slot_key(s0) : 0;
      const int k1 = s0 + 2 < nslots ? slot_key(s0 + 2) : 0;
      if constexpr (sizeof(T) == 2) {
        return u32x4{*reinterpret_cast<const uint32_t*>(vrow + k0),
                     *reinterpret_cast<const uint32_t*>(vrow + k1), 0u, 0u};
      } else {
        const u32x2 a = *reinterpret_cast<const u32x2*>(vrow + k0);
        const u32x2 b = *reinterpret_cast<const u32x2*>(vrow + k1);
        return u32x4{a[0], a[1], b[0], b[1]};
      }
    } else {
      int kk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) kk[e] = s0 + e < nslots ? slot_key(s0 + e) : 0;
      if constexpr (sizeof(T) == 2) {
        const uint32_t e0 = reinterpret_cast<const uint16_t*>(vrow)[kk[0]];
        const uint32_t e1 = reinterpret_cast<const uint16_t*>(vrow)[kk[1]];
        const uint32_t e2 = reinterpret_cast<const uint16_t*>(vrow)[kk[2]];
        const uint32_t e3 = reinterpret_cast<const uint16_t*>(vrow)[kk[3]];
        return u32x4{e0 | (e1 << 16), e2 | (e3 << 16), 0u, 0u};
      } else {
        const uint32_t* vr = reinterpret_cast<const uint32_t*>(vrow);
        return u32x4{vr[kk[0]], vr[kk[1]], vr[kk[2]], vr[kk[3]]};
      }
    }
  };

  auto compute_chunk = [&](int c, int buf) {
    // -- compaction of this wave's mask bits for the chunk's key tiles --
    uint32_t nk = 0;
#pragma unroll
    for (int win = 0; win < C::NWIN; ++win) {
      const uint64_t bits = row_bits(mask_row, c * C::TPC + win * C::WINT, C::WINT, p.T_k);
      nk += wave_compact64(bits, win * C::WINT, nk,
                           [&](uint32_t pos, int val) { tl[pos] = (uint8_t)val; });
    }
    const int nslots = wave_uniform((int)nk * N);
    if (nslots == 0) return;
    __builtin_amdgcn_wave_barrier();

    const T* kl = k_lds[buf];
    const T* vl = vt_lds[buf];
    const int kbase = c * KC;
    const int nsb = (nslots + 15) >> 4;

    for (int p0 = 0; p0 < nsb; p0 += C::PASS_SB) {
      const int nsbp = nsb - p0 < C::PASS_SB ? nsb - p0 : C::PASS_SB;
      f32x4 s[C::PASS_SB];
      // -- S^T = K Q^T for up to PASS_SB blocks of 16 slots --
#pragma unroll
      for (int sb = 0; sb < C::PASS_SB; ++sb) {
        s[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (sb < nsbp) {
          const int slot = (p0 + sb) * 16 + n;
          const int key = slot < nslots ? slot_key(slot) : 0;
          const T* krow = kl + key * C::KSTR + VEC * g;
#pragma unroll
          for (int sl = 0; sl < C::NSLAB; ++sl) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(krow + C::SLAB * sl);
            if constexpr (sizeof(T) == 2) s[sb] = Mma<bf16_t>::mac8(a, qf[sl], s[sb]);
            else s[sb] = Mma<float>::mac4(a, qf[sl], s[sb]);
          }
        }
      }
      // -- mask, scale to log2 domain, running max --
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < C::PASS_SB; ++sb) {
        if (sb < nsbp) {
          const int s0 = (p0 + sb) * 16 + 4 * g;
          // keys left in the sequence after this quad's first key (<= 0: none)
          const int room = N >= 4 ? (s0 < nslots ? L - kbase - slot_key(s0) : 0) : 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            bool ok;
            if constexpr (N >= 4) {
              ok = i < room;
            } else {
              ok = s0 + i < nslots && kbase + slot_key(s0 + i) < L;
            }
            const float t = ok ? s[sb][i] * p.scale_log2 : -INFINITY;
            s[sb][i] = t;
            mx = fmaxf(mx, t);
          }
        }
      }
      mx = fmaxf(mx, xor_lane16(mx));
      mx = fmaxf(mx, xor_lane32(mx));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - m_use);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < C::NDB; ++j) oacc[j] *= alpha;
#pragma unroll
      for (int sb = 0; sb < C::PASS_SB; ++sb) {
        if (sb < nsbp) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e = exp2_fast(s[sb][i] - m_use);
            s[sb][i] = e;
            l_run += e;
          }
        }
      }
      // -- O^T += V^T P^T --
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int pp = 0; pp < C::PASS_SB / 2; ++pp) {
          const int sb0 = 2 * pp, sb1 = 2 * pp + 1;
          if (sb0 < nsbp) {
            const bool has1 = sb1 < nsbp;
            bf16x8 pb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              pb[i] = (__bf16)s[sb0][i];
              pb[4 + i] = (__bf16)(has1 ? s[sb1][i] : 0.f);
            }
            const u32x4 bop = __builtin_bit_cast(u32x4, pb);
            const int sA = (p0 + sb0) * 16 + 4 * g;
            const int sB = has1 ? (p0 + sb1) * 16 + 4 * g : nslots;  // dummy when absent
#pragma unroll
            for (int j = 0; j < C::NDB; ++j) {
              const T* vrow = vl + (16 * j + n) * C::VSTR;
              const u32x4 x0 = vt_quad(vrow, sA, nslots);
              const u32x4 x1 = vt_quad(vrow, sB, nslots);
              const u32x4 a = {x0[0], x0[1], x1[0], x1[1]};
              oacc[j] = Mma<bf16_t>::mac8(a, bop, oacc[j]);
            }
          }
        }
      } else {
#pragma unroll
        for (int sb = 0; sb < C::PASS_SB; ++sb) {
          if (sb < nsbp) {
            const u32x4 bop = __builtin_bit_cast(u32x4, s[sb]);
            const int sA = (p0 + sb) * 16 + 4 * g;
#pragma unroll
            for (int j = 0; j < C::NDB; ++j) {
              const T* vrow = vl + (16 * j + n) * C::VSTR;
              oacc[j] = Mma<float>::mac4(vt_quad(vrow, sA, nslots), bop, oacc[j]);
            }
          }
        }
      }
    }
  };

  // ---- main loop over key chunks (double-buffered LDS) ----
  const int n_chunks = (L + KC - 1) / KC;
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int c = 0; c < n_chunks; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < n_chunks;
    if (more) load_chunk(c + 1);
    if (wave_active) compute_chunk(c, buf);
    if (more) store_chunk(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and store ----
  if (!wave_active) return;
  float l_tot = l_run + xor_lane16(l_run);
  l_tot += xor_lane32(l_tot);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int r = row0 + n;
  if (r < L) {
    T* og = reinterpret_cast<T*>(p.o) + head_off + (size_t)r * D;
#pragma unroll
    for (int j = 0; j < C::NDB; ++j) {
      const f32x4 val = oacc[j] * inv;
      if constexpr (sizeof(T) == 2) {
        bf16x4 ob;
#pragma unroll
        for (int i = 0; i < 4; ++i) ob[i] = (__bf16)val[i];
        *reinterpret_cast<u32x2*>(og + 16 * j + 4 * g) = __builtin_bit_cast(u32x2, ob);
      } else {
        *reinterpret_cast<f32x4*>(og + 16 * j + 4 * g) = val;
      }
    }
    if (p.lse != nullptr && g == 0) {
      p.lse[(size_t)bh * L + r] =
          l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
  }
}

}  // namespace tsa
