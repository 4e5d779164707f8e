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
//     it, so K/V are read from HBM/L2 once per work-group, not once per
//     query tile.
//   * Per chunk each wave compacts its own mask bits into the list of kept
//     key tiles (wave prefix count of the bitmap, the routine the compaction
//     kernel also uses) and packs the kept keys densely into 16-key "slots".
//     Matrix-core work is spent only on kept keys: a skipped tile costs its
//     mask bit, and kept tiles of any width N share MFMA blocks instead of
//     each being padded to 16 keys.
//   * Scores are formed transposed, S^T = K Q^T (A = gathered K rows from LDS,
//     B = the wave's Q fragment held in registers), so each lane owns one
//     query column and the S^T accumulator layout is directly the B operand of
//     O^T += V^T P^T: probabilities never leave registers.
//   * Padding slots need no per-score masking: for QK^T they read a kept key
//     of the same row (so the running max only ever sees real kept scores),
//     for PV they read zero columns of the LDS V^T tile.  Keys past L read as
//     zero V columns as well.  The softmax denominator comes out of the
//     matrix cores too: V^T carries one extra row of ones (zero past L and in
//     the padding columns), so l = P . 1 accumulates with O.
//   * Online softmax in base 2 with scale*log2(e) folded into one FMA per
//     score; the reference max is raised (and O, l rescaled) only when some
//     row's max grows by more than 2^8, a wave-uniform decision, so most
//     passes do no rescaling.  The result O / l is unchanged by the choice of
//     reference.
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
  static constexpr int VPAD = 4;                   // zero columns after the KC keys of a V^T row
  static constexpr int VSTR = KC + VPAD;           // V^T row stride: 264 B (bf16) / 272 B (fp32)
  static constexpr int VROWS = D + 1;              // V^T rows: d = 0..D-1 and the ones row
  static constexpr int ZCOL = KC;                  // first zero column of V^T
  static constexpr int NT = 64 * W;
  static constexpr int CPR = D / VEC;              // 16-byte chunks per K/V row
  static constexpr int K_ITEMS = KC * CPR;
  static constexpr int V_ITEMS = (KC / 4) * CPR;   // groups of 4 rows x 16 bytes
  static constexpr int K_PER_T = (K_ITEMS + NT - 1) / NT;
  static constexpr int V_PER_T = (V_ITEMS + NT - 1) / NT;
  static constexpr int TPC = KC / N;               // key tiles per chunk
  static constexpr int WINT = TPC < 64 ? TPC : 64; // tiles per compaction window
  static constexpr int NWIN = TPC / WINT;
  static constexpr int MW = TPC >= 32 ? TPC / 32 : 1;  // mask words per chunk
  static constexpr int LOG2N = ilog2(N);
  static constexpr int MAXSB = KC / 16;            // 16-slot sub-blocks per chunk
  static_assert(D % SLAB == 0 && D % 16 == 0, "head dim");
  static_assert(KC % N == 0 && KC % 64 == 0 && TPC <= 256 && MW <= 4, "chunk");
  static_assert((1 << LOG2N) == N, "N must be a power of two");
  // V staging: a wave covers 16 consecutive key quads x 4 16-byte d chunks
  static constexpr int VQ = KC / 4;                // key quads per chunk
  static_assert(VQ % 16 == 0 && CPR % 4 == 0, "V staging tile");
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
struct AttnKernel {
  using C = AttnCfg<T, D, N, KC, W>;
  static constexpr int VEC = C::VEC;
  static constexpr float RESCALE_STEP = 8.f;  // log2 units a row max may grow before rescaling

  struct Smem {
    T k[2][KC * C::KSTR];
    T vt[2][C::VROWS * C::VSTR];
    uint8_t tl[W][C::TPC];
  };

  // ---- per-wave state ----
  const AttnParams& p;
  Smem& sm;
  int tid, lane, g, n, wave;
  int L, bh, row0;
  bool active;
  const T* __restrict__ kg;
  const T* __restrict__ vg;
  const uint32_t* __restrict__ mask_row;
  u32x4 qf[C::NSLAB];
  f32x4 oacc[C::NDB + 1];  // O^T blocks and, last, the row sums l
  float m_run;             // reference max (log2 domain) of query n
  u32x4 kreg[C::K_PER_T];
  u32x4 vreg[C::V_PER_T][4];

  __device__ __forceinline__ AttnKernel(const AttnParams& pp, Smem& s) : p(pp), sm(s) {}

  __device__ __forceinline__ int tl_at(int idx) const { return (int)sm.tl[wave][idx]; }

  // V staging item -> (key quad rg, 16-byte d chunk ch).  Lane l of a wave
  // takes quad (l % 16) and chunk (l / 16) of the wave's 16 x 4 block, so the
  // 16 lanes writing one V^T row write 128 contiguous bytes.
  __device__ __forceinline__ void v_item(int idx, int& rg, int& ch) const {
    const int l = idx & 63, blk = idx >> 6;
    constexpr int QB = C::VQ / 16;                 // 16-quad blocks per chunk
    rg = (blk % QB) * 16 + (l & 15);
    ch = (blk / QB) * 4 + (l >> 4);
  }

  // Global -> registers for chunk c (K rows, V rows, this wave's mask words).
  // Full chunks address from a uniform chunk base plus a per-thread constant;
  // the last, partial chunk clamps to row L-1 and zero-fills keys past L.
  __device__ __forceinline__ void load_chunk(int c, uint32_t (&mreg)[C::MW]) {
    const int kbase = c * KC;
    const T* kc_base = kg + (size_t)kbase * D;
    const T* vc_base = vg + (size_t)kbase * D;
    if (kbase + KC <= L) {
#pragma unroll
      for (int u = 0; u < C::K_PER_T; ++u) {
        const int idx = tid + u * C::NT;
        if (C::K_ITEMS % C::NT == 0 || idx < C::K_ITEMS)
          kreg[u] = *reinterpret_cast<const u32x4*>(kc_base + (idx / C::CPR) * D + (idx % C::CPR) * VEC);
      }
#pragma unroll
      for (int u = 0; u < C::V_PER_T; ++u) {
        const int idx = tid + u * C::NT;
        if (C::V_ITEMS % C::NT == 0 || idx < C::V_ITEMS) {
          int rg, ch;
          v_item(idx, rg, ch);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            vreg[u][r] = *reinterpret_cast<const u32x4*>(vc_base + (4 * rg + r) * D + ch * VEC);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < C::K_PER_T; ++u) {
        const int idx = tid + u * C::NT;
        if (C::K_ITEMS % C::NT == 0 || idx < C::K_ITEMS) {
          const int row = idx / C::CPR, ch = idx % C::CPR;
          const int rc = kbase + row < L ? row : L - 1 - kbase;
          kreg[u] = *reinterpret_cast<const u32x4*>(kc_base + rc * D + ch * VEC);
          if (kbase + row >= L) kreg[u] = u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < C::V_PER_T; ++u) {
        const int idx = tid + u * C::NT;
        if (C::V_ITEMS % C::NT == 0 || idx < C::V_ITEMS) {
          int rg, ch;
          v_item(idx, rg, ch);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 4 * rg + r;
            const int rc = kbase + row < L ? row : L - 1 - kbase;
            vreg[u][r] = *reinterpret_cast<const u32x4*>(vc_base + rc * D + ch * VEC);
            if (kbase + row >= L) vreg[u][r] = u32x4{0u, 0u, 0u, 0u};
          }
        }
      }
    }
    // mask words holding key tiles [c*TPC, c*TPC + TPC) of this wave's row
    const int w0 = (c * C::TPC) >> 5;
#pragma unroll
    for (int i = 0; i < C::MW; ++i) {
      const int wi = w0 + i < p.words ? w0 + i : p.words - 1;
      mreg[i] = mask_row[wi];
    }
  }

  // Registers -> LDS buffer `buf` for chunk c (V transposed; ones row).
  __device__ __forceinline__ void store_chunk(int c, int buf) {
#pragma unroll
    for (int u = 0; u < C::K_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      if (C::K_ITEMS % C::NT == 0 || idx < C::K_ITEMS) {
        const int row = idx / C::CPR, ch = idx % C::CPR;
        *reinterpret_cast<u32x4*>(&sm.k[buf][row * C::KSTR + ch * VEC]) = kreg[u];
      }
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_T; ++u) {
      const int idx = tid + u * C::NT;
      if (C::V_ITEMS % C::NT == 0 || idx < C::V_ITEMS) {
        int rg, ch;
        v_item(idx, rg, ch);
        T* dst = &sm.vt[buf][(ch * VEC) * C::VSTR + 4 * rg];
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
    // ones row: 1 for keys < L, 0 past L
    if (tid < KC / VEC) {
      const int k0 = c * KC + tid * VEC;
      u32x4 v;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo = k0 + 2 * w < L ? 0x3f80u : 0u;
          const uint32_t hi = k0 + 2 * w + 1 < L ? 0x3f800000u : 0u;
          v[w] = lo | hi;
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) v[w] = k0 + w < L ? 0x3f800000u : 0u;
      }
      *reinterpret_cast<u32x4*>(&sm.vt[buf][D * C::VSTR + tid * VEC]) = v;
    }
  }

  // Zero the V^T padding columns (read by padding slots) of both buffers.
  __device__ __forceinline__ void zero_pad_columns() {
    for (int r = tid; r < 2 * C::VROWS; r += C::NT) {
      const int buf = r / C::VROWS, row = r % C::VROWS;
      T* dst = &sm.vt[buf][row * C::VSTR + KC];
      if constexpr (sizeof(T) == 2) *reinterpret_cast<u32x2*>(dst) = u32x2{0u, 0u};
      else *reinterpret_cast<u32x4*>(dst) = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // Four consecutive V^T elements for slots s0..s0+3 (N >= 4: one read).
  // FULL: every slot is known to be < nslots.
  template <bool FULL>
  __device__ __forceinline__ u32x2 vt_quad_b16(const T* vrow, int s0, int nslots) const {
    if constexpr (FULL) nslots = 0x7fffffff;
    if constexpr (N >= 4) {
      const int s = s0 < nslots ? s0 : 0;
      const int kk = (tl_at(s >> C::LOG2N) << C::LOG2N) | (s & (N - 1));
      return *reinterpret_cast<const u32x2*>(vrow + (s0 < nslots ? kk : C::ZCOL));
    } else if constexpr (N == 2) {
      int kk[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int s = s0 + 2 * e;
        const int t = tl_at(s < nslots ? (s >> 1) : 0) << 1;
        kk[e] = s < nslots ? t : C::ZCOL;
      }
      return u32x2{*reinterpret_cast<const uint32_t*>(vrow + kk[0]),
                   *reinterpret_cast<const uint32_t*>(vrow + kk[1])};
    } else {
      uint32_t e4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = s0 + e;
        const int t = tl_at(s < nslots ? s : 0);
        e4[e] = reinterpret_cast<const uint16_t*>(vrow)[s < nslots ? t : C::ZCOL];
      }
      return u32x2{e4[0] | (e4[1] << 16), e4[2] | (e4[3] << 16)};
    }
  }

  template <bool FULL>
  __device__ __forceinline__ u32x4 vt_quad_f32(const T* vrow, int s0, int nslots) const {
    if constexpr (FULL) nslots = 0x7fffffff;
    if constexpr (N >= 4) {
      const int s = s0 < nslots ? s0 : 0;
      const int kk = (tl_at(s >> C::LOG2N) << C::LOG2N) | (s & (N - 1));
      return *reinterpret_cast<const u32x4*>(vrow + (s0 < nslots ? kk : C::ZCOL));
    } else if constexpr (N == 2) {
      u32x2 a[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int s = s0 + 2 * e;
        const int t = tl_at(s < nslots ? (s >> 1) : 0) << 1;
        a[e] = *reinterpret_cast<const u32x2*>(vrow + (s < nslots ? t : C::ZCOL));
      }
      return u32x4{a[0][0], a[0][1], a[1][0], a[1][1]};
    } else {
      u32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = s0 + e;
        const int t = tl_at(s < nslots ? s : 0);
        r[e] = reinterpret_cast<const uint32_t*>(vrow)[s < nslots ? t : C::ZCOL];
      }
      return r;
    }
  }

  // One softmax pass over NSB sub-blocks of 16 slots starting at sub-block sb0.
  // FULL: all slots of the pass are < nslots and every key of the chunk is < L.
  template <int NSB, bool FULL>
  __device__ __forceinline__ void pass(const T* kl, const T* vl, int sb0, int nslots, int lim,
                                       int key0) {
    if constexpr (FULL) {
      nslots = 0x7fffffff;
      lim = 0x7fffffff;
    }
    // QK^T A rows: a padding slot reads the first kept key; a key past L the
    // start of its (kept) tile.  Either way the score is a real kept score.
    int ka[NSB];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      const int slot = 16 * (sb0 + sb) + n;
      const int sc = slot < nslots ? slot : 0;
      const int t = tl_at(sc >> C::LOG2N) << C::LOG2N;
      int key = t | (sc & (N - 1));
      key = key < lim ? key : t;
      key = slot < nslots ? key : key0;
      ka[sb] = key * C::KSTR + VEC * g;
    }
    f32x4 s[NSB];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) s[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sl = 0; sl < C::NSLAB; ++sl) {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kl + ka[sb] + C::SLAB * sl);
        if constexpr (sizeof(T) == 2) s[sb] = Mma<bf16_t>::mac8(a, qf[sl], s[sb]);
        else s[sb] = Mma<float>::mac4(a, qf[sl], s[sb]);
      }
    }
    // running max in the log2 domain (scale may be negative)
    const float c = p.scale_log2;
    float mr = s[0][0];
    if (c >= 0.f) {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mr = fmaxf(mr, s[sb][i]);
    } else {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mr = fminf(mr, s[sb][i]);
    }
    float mx = c * mr;
    mx = fmaxf(mx, xor_lane16(mx));
    mx = fmaxf(mx, xor_lane32(mx));
    if (__builtin_amdgcn_ballot_w64(mx > m_run + RESCALE_STEP) != 0ull) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2_fast(m_run - m_new);  // 0 on the first pass
      m_run = m_new;
#pragma unroll
      for (int j = 0; j <= C::NDB; ++j) oacc[j] *= alpha;
    }
    const float nm = -m_run;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[sb][i] = exp2_fast(__builtin_fmaf(s[sb][i], c, nm));
    // O^T += V^T P^T (and l += P . 1 through the ones row)
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int pp = 0; pp < (NSB + 1) / 2; ++pp) {
        const int a0 = 2 * pp, a1 = 2 * pp + 1;
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[i] = (__bf16)s[a0][i];
          pb[4 + i] = a1 < NSB ? (__bf16)s[a1 < NSB ? a1 : a0][i] : (__bf16)0.f;
        }
        const u32x4 bop = __builtin_bit_cast(u32x4, pb);
        const int sA = 16 * (sb0 + a0) + 4 * g;
        const int sB = 16 * (sb0 + a1) + 4 * g;
#pragma unroll
        for (int j = 0; j <= C::NDB; ++j) {
          const T* vrow = vl + (j < C::NDB ? 16 * j + n : D) * C::VSTR;
          const u32x2 x0 = vt_quad_b16<FULL>(vrow, sA, nslots);
          const u32x2 x1 = a1 < NSB ? vt_quad_b16<FULL>(vrow, sB, nslots)
                                    : *reinterpret_cast<const u32x2*>(vrow + C::ZCOL);
          oacc[j] = Mma<bf16_t>::mac8(u32x4{x0[0], x0[1], x1[0], x1[1]}, bop, oacc[j]);
        }
      }
    } else {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const u32x4 bop = __builtin_bit_cast(u32x4, s[sb]);
        const int sA = 16 * (sb0 + sb) + 4 * g;
#pragma unroll
        for (int j = 0; j <= C::NDB; ++j) {
          const T* vrow = vl + (j < C::NDB ? 16 * j + n : D) * C::VSTR;
          oacc[j] = Mma<float>::mac4(vt_quad_f32<FULL>(vrow, sA, nslots), bop, oacc[j]);
        }
      }
    }
  }

  __device__ __forceinline__ void compute_chunk(int c, int buf, const uint32_t (&mreg)[C::MW]) {
    // -- compaction of this wave's mask bits for the chunk's key tiles --
    const int first = c * C::TPC;
    uint32_t nk = 0;
#pragma unroll
    for (int win = 0; win < C::NWIN; ++win) {
      uint64_t bits;
      if constexpr (C::WINT == 64) {
        bits = (uint64_t)uniform_u32(mreg[2 * win]) | ((uint64_t)uniform_u32(mreg[2 * win + 1]) << 32);
      } else {
        const uint32_t w = uniform_u32(mreg[0]) >> (first & 31);
        bits = C::WINT == 32 ? (uint64_t)w : (uint64_t)(w & ((1u << C::WINT) - 1u));
      }
      const int room = p.T_k - first - win * C::WINT;  // valid tiles left in the row
      if (room < C::WINT) bits = room <= 0 ? 0ull : (bits & ((1ull << room) - 1ull));
      nk += wave_compact64(bits, win * C::WINT, nk,
                           [&](uint32_t pos, int val) { sm.tl[wave][pos] = (uint8_t)val; });
    }
    const int nslots = (int)nk * N;
    if (nslots == 0) return;
    __builtin_amdgcn_wave_barrier();
    const T* kl = sm.k[buf];
    const T* vl = sm.vt[buf];
    const int lim = L - c * KC;              // keys of this chunk that exist
    const int key0 = tl_at(0) << C::LOG2N;   // first kept key of the chunk
    const int nsb = (nslots + 15) >> 4;
    const bool full_chunk = lim >= KC;
    int sb0 = 0;
    for (; sb0 + 4 <= nsb; sb0 += 4) {
      if (full_chunk && 16 * (sb0 + 4) <= nslots) pass<4, true>(kl, vl, sb0, nslots, lim, key0);
      else pass<4, false>(kl, vl, sb0, nslots, lim, key0);
    }
    const int rem = nsb - sb0;
    const bool full_tail = full_chunk && (nslots & 15) == 0;
    if (rem == 3) {
      if (full_tail) pass<3, true>(kl, vl, sb0, nslots, lim, key0);
      else pass<3, false>(kl, vl, sb0, nslots, lim, key0);
    } else if (rem == 2) {
      if (full_tail) pass<2, true>(kl, vl, sb0, nslots, lim, key0);
      else pass<2, false>(kl, vl, sb0, nslots, lim, key0);
    } else if (rem == 1) {
      if (full_tail) pass<1, true>(kl, vl, sb0, nslots, lim, key0);
      else pass<1, false>(kl, vl, sb0, nslots, lim, key0);
    }
  }

  __device__ __forceinline__ void run() {
    tid = threadIdx.x;
    lane = tid & 63;
    g = lane >> 4;
    n = lane & 15;
    wave = wave_uniform(tid >> 6);
    bh = blockIdx.x / p.n_qblocks;
    const int qb = blockIdx.x - bh * p.n_qblocks;
    L = p.L;
    const size_t head_off = (size_t)bh * (size_t)L * D;
    const T* __restrict__ qg = reinterpret_cast<const T*>(p.q) + head_off;
    kg = reinterpret_cast<const T*>(p.k) + head_off;
    vg = reinterpret_cast<const T*>(p.v) + head_off;
    row0 = qb * (16 * W) + 16 * wave;
    active = row0 < L;
    const int mrow = active ? row0 / p.M : 0;
    mask_row = p.mask + ((size_t)bh * p.T_q + (size_t)mrow) * p.words;

    // Q fragment: lane (g, n) holds Q[row0+n][SLAB*s + VEC*g .. +VEC)
    {
      const int r = row0 + n < L ? row0 + n : L - 1;
#pragma unroll
      for (int s = 0; s < C::NSLAB; ++s)
        qf[s] = *reinterpret_cast<const u32x4*>(qg + (size_t)r * D + C::SLAB * s + VEC * g);
      if (row0 + n >= L)
#pragma unroll
        for (int s = 0; s < C::NSLAB; ++s) qf[s] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j <= C::NDB; ++j) oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;

    zero_pad_columns();
    const int n_chunks = (L + KC - 1) / KC;
    uint32_t mcur[C::MW], mnext[C::MW];
    load_chunk(0, mcur);
    store_chunk(0, 0);
    __syncthreads();
    for (int c = 0; c < n_chunks; ++c) {
      const int buf = c & 1;
      const bool more = c + 1 < n_chunks;
      if (more) load_chunk(c + 1, mnext);
      if (active) compute_chunk(c, buf, mcur);
      if (more) {
        store_chunk(c + 1, buf ^ 1);
#pragma unroll
        for (int i = 0; i < C::MW; ++i) mcur[i] = mnext[i];
      }
      __syncthreads();
    }

    // normalise and store
    if (!active) return;
    const float l_tot = oacc[C::NDB][0];
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
};

template <typename T, int D, int N, int KC, int W>
__global__ __launch_bounds__(64 * W) void attn_fwd_kernel(AttnParams p) {
  using K = AttnKernel<T, D, N, KC, W>;
  __shared__ __attribute__((aligned(16))) typename K::Smem sm;
  K k(p, sm);
  k.run();
}

}  // namespace tsa
