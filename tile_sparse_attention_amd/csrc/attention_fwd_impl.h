// Tile-sparse attention forward kernel (gfx950, wave64, MFMA).
//
// Operation: FG-Attn ("FG-Attn: Leveraging Fine-Grained Sparse Attention in
// Video Diffusion Models", section Abstract) skips the query-key dot products
// of every M x N tile whose keep bit is 0 and leaves those scores out of the
// softmax.  O = softmax(scale * Q K^T restricted to kept tiles) V.
//
// Work decomposition
//   * A work-group owns 32*W consecutive query rows of one (b, h); each wave
//     owns 32 of them as two 16-row query tiles (M is a multiple of 16, so a
//     16-row tile lies inside one mask row).
//   * Keys are streamed in chunks of KC keys.  The work-group stages each
//     chunk once in LDS (K as rows, V transposed to [d][key]) with
//     double-buffered buffer loads whose chunk offset is a uniform value; all
//     waves then reuse it, so each K/V element crosses from L2 once per
//     32*W query rows.  Blocks are renumbered so that the work-groups running
//     together on one XCD belong to one head and stream the same K/V through
//     that XCD's L2.
//   * Per chunk each wave compacts its mask bits into the list of kept key
//     tiles (wave prefix count of the bitmap, the routine the compaction
//     kernel also uses) and packs the kept keys densely into 16-key "slots":
//     matrix-core work is spent only on kept keys, and kept tiles of any
//     width N share MFMA blocks instead of each being padded to 16 keys.
//     When M >= 32 both query tiles of a wave lie in the same mask row and
//     share one compacted list.
//   * Scores are formed transposed, S^T = K Q^T (A = gathered K rows from LDS,
//     B = the tile's Q fragment held in registers), so each lane owns one
//     query column and the S^T accumulator layout is directly the B operand of
//     O^T += V^T P^T: probabilities never leave registers.  For N >= 8 the
//     rows of each pair of 16-slot blocks are assigned to slots so that every
//     lane's eight PV k-values are eight consecutive keys: one 16-byte LDS
//     read per MFMA operand.
//   * Padding slots need no per-score masking: for QK^T they read a kept key
//     of the same row (so the running max only ever sees real kept scores),
//     for PV they read zero columns of the LDS V^T tile.  Keys past L read as
//     zero V columns as well.  The softmax denominator comes out of the
//     matrix cores too: V^T carries one extra row of ones (zero past L and in
//     the padding columns), so l = P . 1 accumulates with O.
//   * Online softmax in base 2 with scale*log2(e) folded into one FMA per
//     score.  The reference max is raised (and O, l rescaled) only when some
//     lane's scores exceed it by more than 2^8, a wave-uniform ballot, so most
//     passes do neither a cross-lane reduction nor a rescale.  The result
//     O / l does not depend on the choice of reference.
//   * Normalisation O = O / l (0 for a row with nothing kept) and the store
//     happen once at the end.
#pragma once

#include "tsa_device.h"

namespace tsa {

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;         // V [B*H][L][d] (read as rows by the key-packing kernel)
  const void* vt;        // packed V^T: [B*H][d + 1][L_pad], row d = ones (keys < L)
  const uint32_t* mask;
  void* o;
  float* lse;
  int H, L, M, T_q, T_k, words;
  int L_pad;             // row length of the packed V^T (multiple of 128)
  int n_qblocks;
  float scale_log2;  // scale * log2(e)
  // chunk skipping (octet kernel): per work-group, kNeedWords bitmap words
  // of needed chunks, one flag word per work-group, and the number of
  // flagged work-groups (null: no skipping)
  const uint32_t* need;
  const uint32_t* need_flag;
  const uint32_t* need_count;
  // FP8 scores (q and k hold e4m3 bytes): per (b, h) ceil(L/16) Q tile scales
  // and one K scale (null otherwise)
  const float* q_scale;
  const float* k_scale;
};

template <typename T> struct ElemTraits;
template <> struct ElemTraits<float> { static constexpr int VEC = 4; };
template <> struct ElemTraits<bf16_t> { static constexpr int VEC = 8; };

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }


template <typename T, int D, int N, int KC, int W, int TPW>
struct AttnCfg {
  static constexpr int VEC = ElemTraits<T>::VEC;   // elements per 16 bytes
  static constexpr int SLAB = 4 * VEC;             // d covered by one 16-byte read per lane group
  static constexpr int NSLAB = D / SLAB;
  static constexpr int NDB = D / 16;               // 16-wide d blocks of O^T
  static constexpr int KSTR = D + VEC;             // K row stride in LDS (+16 B against bank conflicts)
  static constexpr int VPAD = VEC;                 // zero columns after the KC keys of a V^T row
  static constexpr int VSTR = KC + VPAD;           // V^T row stride (272 B for bf16, KC = 128)
  static constexpr int VROWS = D + 1;              // V^T rows: d = 0..D-1 and the ones row
  static constexpr int ZCOL = KC;                  // first zero column of V^T
  static constexpr int NT = 64 * W;
  static constexpr int ROWS = 16 * TPW * W;        // query rows per work-group
  static constexpr int CPR = D / VEC;              // 16-byte chunks per K/V row
  static constexpr int TPC = KC / N;               // key tiles per chunk
  static constexpr int WINT = TPC < 64 ? TPC : 64; // tiles per compaction window
  static constexpr int NWIN = TPC / WINT;
  static constexpr int MW = TPC >= 32 ? TPC / 32 : 1;  // mask words per chunk
  static constexpr int LOG2N = ilog2(N);
  // bf16 with N >= 8: pairs of 16-slot blocks use the octet slot order
  static constexpr bool OCT = sizeof(T) == 2 && N >= 8;
  // LDS tiles are filled by direct global->LDS loads: one wave instruction
  // writes 1 KB (16 bytes per lane) contiguously, so a tile of padded rows is
  // covered by whole 1-KB instructions; lanes that land on row padding (or
  // past the last row) read out of range and write zeros.
  static constexpr int KRB = D * (int)sizeof(T);          // K row bytes in memory
  static constexpr int KRS = KSTR * (int)sizeof(T);       // K row stride in LDS
  static constexpr int VRB = KC * (int)sizeof(T);         // V^T row bytes per chunk
  static constexpr int VRS = VSTR * (int)sizeof(T);       // V^T row stride in LDS
  static constexpr int NI_K = (KC * KRS + 1023) / 1024;   // 1-KB loads per K tile
  static constexpr int NI_V = (VROWS * VRS + 1023) / 1024;
  static constexpr int NI = NI_K + NI_V;
  static constexpr int NI_W = (NI + W - 1) / W;           // loads per wave per chunk
  static_assert(D % SLAB == 0 && D % 16 == 0, "head dim");
  static_assert(KC % N == 0 && KC % 64 == 0 && TPC <= 256 && MW <= 4, "chunk");
  static_assert((1 << LOG2N) == N, "N must be a power of two");
  static_assert(KRS == KRB + 16 && VRS == VRB + 16, "one 16-byte padding slot per row");
};

template <typename T> struct Mma;

// One 16x16x128 FP8 (e4m3) matrix-core step, block scales 2^0: lane (g, n)
// supplies 32 bytes of A's row n and of B's column n (a0|a1, b0|b1), the
// same 32 k positions of the contraction in both.
__device__ __forceinline__ f32x4 mac_fp8(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x4 c) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

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

template <typename T, int D, int N, int KC, int W, int TPW>
struct AttnKernel {
  using C = AttnCfg<T, D, N, KC, W, TPW>;
  static constexpr int VEC = C::VEC;
  static constexpr float RESCALE_STEP = 8.f;  // log2 units a row max may grow before rescaling
  // With four waves per SIMD (one tile per wave) the register budget is 128:
  // loads of a pass are then not all hoisted ahead of their MFMAs; the other
  // waves hide the latency instead.
  static constexpr bool LIMIT_ILP = TPW == 1;

  struct Smem {
    __attribute__((aligned(16))) T k[2][C::NI_K * 1024 / sizeof(T)];
    __attribute__((aligned(16))) T vt[2][C::NI_V * 1024 / sizeof(T)];
    uint8_t tl[W][TPW][C::TPC];
  };

  // per-tile state (a wave owns TPW 16-row query tiles)
  struct Tile {
    u32x4 qf[C::NSLAB];       // Q fragment: lane (g, n) holds Q[row+n][SLAB*s + VEC*g .. +VEC)
    f32x4 oacc[C::NDB + 1];   // O^T blocks and, last, the row sums l
    float m_run;              // reference max (log2 domain) of query n
  };

  const AttnParams& p;
  Smem& sm;
  int tid, lane, g, n, wave;
  int L, bh, row0;
  const T* __restrict__ kg;
  const T* __restrict__ vtg;
  const uint32_t* __restrict__ mask_row[TPW];
  Tile tile[TPW];

  __device__ __forceinline__ AttnKernel(const AttnParams& pp, Smem& s) : p(pp), sm(s) {}

  __device__ __forceinline__ int tl_at(int list, int idx) const {
    return (int)sm.tl[wave][list][idx];
  }

  // Byte offset (relative to the chunk's resource base) that lane `ln` of
  // tile load `I` reads, or an out-of-range offset for padding slots.
  __device__ __forceinline__ uint32_t dma_offset(int I, int ln) const {
    // past every resource's range: an fp32 V^T resource spans up to
    // 129 x 2^22 x 4 bytes, more than 2^31
    constexpr uint32_t OOB = 0xfffffff0u;
    if (I < C::NI_K) {
      const int pos = I * 1024 + 16 * ln;
      const int row = pos / C::KRS, cb = pos - row * C::KRS;
      return row < KC && cb < C::KRB ? (uint32_t)(row * C::KRB + cb) : OOB;
    }
    const int pos = (I - C::NI_K) * 1024 + 16 * ln;
    const int row = pos / C::VRS, cb = pos - row * C::VRS;
    return row < C::VROWS && cb < C::VRB
               ? (uint32_t)row * (uint32_t)p.L_pad * (uint32_t)sizeof(T) + (uint32_t)cb
               : OOB;
  }

  // Issue the direct global->LDS loads of chunk c into buffer `buf` (this
  // wave's share) and the loads of both tiles' mask words for it.  Nothing
  // waits here: the caller waits for the vector-memory counter and syncs the
  // work-group before the buffer is read.
  __device__ __forceinline__ void issue_chunk(int c, int buf, uint32_t (&mreg)[TPW][C::MW]) {
    const int kbase = c * KC;
    const int rows = L - kbase < KC ? L - kbase : KC;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kg + (size_t)kbase * D), (short)0, rows * C::KRB, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vtg + kbase), (short)0, (int)((uint32_t)(C::VROWS * p.L_pad - kbase) * (uint32_t)sizeof(T)),
        kBufferFlags);
    // The per-lane offsets are loop-invariant; recomputing them (a few VALU
    // per load) keeps them out of the register budget instead of holding or
    // spilling them across the chunk loop.
    const int ln = lane + opaque_zero();
#pragma unroll
    for (int u = 0; u < C::NI_W; ++u) {
      const int I = wave + W * u;
      if (C::NI % W == 0 || I < C::NI) {
        if (I < C::NI_K) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rk, (__attribute__((address_space(3))) void*)((char*)sm.k[buf] + I * 1024), 16,
              dma_offset(I, ln), 0, 0, 0);
        } else {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rv, (__attribute__((address_space(3))) void*)((char*)sm.vt[buf] + (I - C::NI_K) * 1024),
              16, dma_offset(I, ln), 0, 0, 0);
        }
      }
    }
    // mask words holding key tiles [c*TPC, c*TPC + TPC) of each tile's row
    const int w0 = (c * C::TPC) >> 5;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i = 0; i < C::MW; ++i) {
        const int wi = w0 + i < p.words ? w0 + i : p.words - 1;
        mreg[t][i] = mask_row[t][wi];
      }
  }

  // key offset (in the chunk) of slot s of list `li`
  __device__ __forceinline__ int slot_key(int li, int s) const {
    if constexpr (N == 1) return tl_at(li, s);
    else return (tl_at(li, s >> C::LOG2N) << C::LOG2N) | (s & (N - 1));
  }

  // Four consecutive slots s0..s0+3 of V^T row `vrow` as a 4-element quad
  // (8 bytes for bf16, 16 bytes for fp32).  FULL: every slot is < nslots.
  template <bool FULL>
  __device__ __forceinline__ u32x4 vt_quad(const T* vrow, int li, int s0, int nslots) const {
    if constexpr (FULL) nslots = 0x7fffffff;
    if constexpr (N >= 4) {
      const int s = s0 < nslots ? s0 : 0;
      const int col = s0 < nslots ? slot_key(li, s) : C::ZCOL;
      if constexpr (sizeof(T) == 2) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(vrow + col);
        return u32x4{x[0], x[1], 0u, 0u};
      } else {
        return *reinterpret_cast<const u32x4*>(vrow + col);
      }
    } else if constexpr (N == 2) {
      int col[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int s = s0 + 2 * e;
        const int t = tl_at(li, s < nslots ? (s >> 1) : 0) << 1;
        col[e] = s < nslots ? t : C::ZCOL;
      }
      if constexpr (sizeof(T) == 2) {
        return u32x4{*reinterpret_cast<const uint32_t*>(vrow + col[0]),
                     *reinterpret_cast<const uint32_t*>(vrow + col[1]), 0u, 0u};
      } else {
        const u32x2 a = *reinterpret_cast<const u32x2*>(vrow + col[0]);
        const u32x2 b = *reinterpret_cast<const u32x2*>(vrow + col[1]);
        return u32x4{a[0], a[1], b[0], b[1]};
      }
    } else {
      uint32_t e4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = s0 + e;
        const int t = tl_at(li, s < nslots ? s : 0);
        const int col = s < nslots ? t : C::ZCOL;
        if constexpr (sizeof(T) == 2) e4[e] = reinterpret_cast<const uint16_t*>(vrow)[col];
        else e4[e] = reinterpret_cast<const uint32_t*>(vrow)[col];
      }
      if constexpr (sizeof(T) == 2) return u32x4{e4[0] | (e4[1] << 16), e4[2] | (e4[3] << 16), 0u, 0u};
      else return u32x4{e4[0], e4[1], e4[2], e4[3]};
    }
  }

  // Eight consecutive slots s0..s0+7 (octet order, N >= 8: one 16-byte read).
  template <bool FULL>
  __device__ __forceinline__ u32x4 vt_oct(const T* vrow, int li, int s0, int nslots) const {
    if constexpr (FULL) nslots = 0x7fffffff;
    const int s = s0 < nslots ? s0 : 0;
    const int col = s0 < nslots ? slot_key(li, s) : C::ZCOL;
    return *reinterpret_cast<const u32x4*>(vrow + col);
  }

  // Running-max update for one tile from its NSB score blocks (raw units),
  // then p = exp2(scale*log2(e)*s - m) in place.
  template <int NSB>
  __device__ __forceinline__ void softmax_tile(Tile& tt, f32x4 (&s)[NSB]) {
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
    // Rescale only if some lane's scores exceed its reference by more than
    // RESCALE_STEP; the new reference is then the row max across the lane
    // groups holding the same query.
    float mx = c * mr;
    if (__builtin_amdgcn_ballot_w64(mx > tt.m_run + RESCALE_STEP) != 0ull) {
      mx = fmaxf(mx, xor_lane16(mx));
      mx = fmaxf(mx, xor_lane32(mx));
      const float m_new = fmaxf(tt.m_run, mx);
      const float alpha = exp2_fast(tt.m_run - m_new);  // 0 on the first pass
      tt.m_run = m_new;
#pragma unroll
      for (int j = 0; j <= C::NDB; ++j) tt.oacc[j] *= alpha;
    }
    const float nm = -tt.m_run;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[sb][i] = exp2_fast(__builtin_fmaf(s[sb][i], c, nm));
  }

  // One pass of tile TA over NSB 16-slot blocks of list `li` starting at
  // block sb0.  FULL: all slots of the pass are < nslots and every key of the
  // chunk is < L.
  template <int NSB, bool FULL, int TA>
  __device__ __forceinline__ void pass(const T* kl, const T* vl, int li, int sb0, int nslots,
                                       int lim, int key0) {
    if constexpr (FULL) {
      nslots = 0x7fffffff;
      lim = 0x7fffffff;
    }
    constexpr int NPAIR = C::OCT ? NSB / 2 : 0;   // blocks 0..2*NPAIR-1 use the octet order
    const int base = 16 * sb0;
    // QK^T A rows: a padding slot reads the first kept key; a key past L the
    // start of its (kept) tile.  Either way the score is a real kept score.
    int ka[NSB];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      int slot;
      if (sb < 2 * NPAIR) slot = base + 32 * (sb >> 1) + 8 * (n >> 2) + 4 * (sb & 1) + (n & 3);
      else slot = base + 16 * sb + n;
      const int sc = slot < nslots ? slot : 0;
      const int t = tl_at(li, sc >> C::LOG2N) << C::LOG2N;
      int key = t | (sc & (N - 1));
      key = key < lim ? key : t;
      key = slot < nslots ? key : key0;
      ka[sb] = key * C::KSTR + VEC * g;
    }
    Tile& tt = tile[TA];
    f32x4 s[NSB];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) s[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sl = 0; sl < C::NSLAB; ++sl) {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kl + ka[sb] + C::SLAB * sl);
        if constexpr (sizeof(T) == 2) s[sb] = Mma<bf16_t>::mac8(a, tt.qf[sl], s[sb]);
        else s[sb] = Mma<float>::mac4(a, tt.qf[sl], s[sb]);
      }
      if constexpr (LIMIT_ILP) __builtin_amdgcn_sched_barrier(0);
    }
    softmax_tile<NSB>(tt, s);
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
        const bool oct = pp < NPAIR;
        const int sO = base + 32 * pp + 8 * g;          // octet order
        const int sA = base + 16 * a0 + 4 * g;          // quad order
        const int sB = base + 16 * a1 + 4 * g;
#pragma unroll
        for (int j = 0; j <= C::NDB; ++j) {
          const T* vrow = vl + (j < C::NDB ? 16 * j + n : D) * C::VSTR;
          u32x4 av;
          if (oct) {
            av = vt_oct<FULL>(vrow, li, sO, nslots);
          } else {
            const u32x4 x0 = vt_quad<FULL>(vrow, li, sA, nslots);
            u32x4 x1;
            if (a1 < NSB) x1 = vt_quad<FULL>(vrow, li, sB, nslots);
            else x1 = *reinterpret_cast<const u32x4*>(vrow + C::ZCOL);
            av = u32x4{x0[0], x0[1], x1[0], x1[1]};
          }
          tt.oacc[j] = Mma<bf16_t>::mac8(av, bop, tt.oacc[j]);
          if constexpr (LIMIT_ILP) {
            if (j % 3 == 2) __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    } else {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const int sA = base + 16 * sb + 4 * g;
#pragma unroll
        for (int j = 0; j <= C::NDB; ++j) {
          const T* vrow = vl + (j < C::NDB ? 16 * j + n : D) * C::VSTR;
          const u32x4 av = vt_quad<FULL>(vrow, li, sA, nslots);
          tt.oacc[j] = Mma<float>::mac4(av, __builtin_bit_cast(u32x4, s[sb]), tt.oacc[j]);
        }
      }
    }
  }

  // Compact mask list `li` for chunk c from its mask words; returns slots.
  __device__ __forceinline__ int compact(int li, int c, const uint32_t (&mw)[C::MW]) {
    const int first = c * C::TPC;
    uint32_t nk = 0;
#pragma unroll
    for (int win = 0; win < C::NWIN; ++win) {
      uint64_t bits;
      if constexpr (C::WINT == 64) {
        bits = (uint64_t)uniform_u32(mw[2 * win]) | ((uint64_t)uniform_u32(mw[2 * win + 1]) << 32);
      } else {
        const uint32_t w = uniform_u32(mw[0]) >> (first & 31);
        bits = C::WINT == 32 ? (uint64_t)w : (uint64_t)(w & ((1u << C::WINT) - 1u));
      }
      const int room = p.T_k - first - win * C::WINT;  // valid tiles left in the row
      if (room < C::WINT) bits = room <= 0 ? 0ull : (bits & ((1ull << room) - 1ull));
      nk += wave_compact64(bits, win * C::WINT, nk,
                           [&](uint32_t pos, int val) { sm.tl[wave][li][pos] = (uint8_t)val; });
    }
    __builtin_amdgcn_wave_barrier();
    return (int)nk * N;
  }

  // Passes of tile TA over the nslots slots of list `li`: blocks of PASS
  // 16-slot sub-blocks, then one shorter pass for the rest.
  template <int TA>
  __device__ __forceinline__ void run_list(const T* kl, const T* vl, int li, int nslots, int lim) {
    constexpr int PASS = 2;
    const int key0 = tl_at(li, 0) << C::LOG2N;   // first kept key of the chunk
    const int nsb = (nslots + 15) >> 4;
    const bool full_chunk = lim >= KC;
    int sb0 = 0;
    for (; sb0 + PASS <= nsb; sb0 += PASS) {
      if (full_chunk && 16 * (sb0 + PASS) <= nslots)
        pass<PASS, true, TA>(kl, vl, li, sb0, nslots, lim, key0);
      else
        pass<PASS, false, TA>(kl, vl, li, sb0, nslots, lim, key0);
    }
    const int rem = nsb - sb0;
    const bool full_tail = full_chunk && (nslots & 15) == 0;
    if constexpr (PASS > 3) {
      if (rem == 3) {
        if (full_tail) pass<3, true, TA>(kl, vl, li, sb0, nslots, lim, key0);
        else pass<3, false, TA>(kl, vl, li, sb0, nslots, lim, key0);
      }
    }
    if constexpr (PASS > 2) {
      if (rem == 2) {
        if (full_tail) pass<2, true, TA>(kl, vl, li, sb0, nslots, lim, key0);
        else pass<2, false, TA>(kl, vl, li, sb0, nslots, lim, key0);
      }
    }
    if (rem == 1) {
      if (full_tail) pass<1, true, TA>(kl, vl, li, sb0, nslots, lim, key0);
      else pass<1, false, TA>(kl, vl, li, sb0, nslots, lim, key0);
    }
  }

  // With two tiles per wave both lie in one mask row when M >= 32 (row0 is
  // a multiple of 32) and share one compacted list; the passes stay per tile
  // (running both tiles through one pass needs more registers than two waves
  // per SIMD leave).
  __device__ __forceinline__ void compute_chunk(int c, int buf, const uint32_t (&mw)[TPW][C::MW],
                                                bool same_row, bool act1) {
    const T* kl = sm.k[buf];
    const T* vl = sm.vt[buf];
    const int lim = L - c * KC;  // keys of this chunk that exist
    const int n0 = compact(0, c, mw[0]);
    if (n0 > 0) run_list<0>(kl, vl, 0, n0, lim);
    if constexpr (TPW == 2) {
      const int l1 = same_row ? 0 : 1;
      const int n1 = !act1 ? 0 : same_row ? n0 : compact(1, c, mw[1]);
      if (n1 > 0) run_list<1>(kl, vl, l1, n1, lim);
    }
  }

  __device__ __forceinline__ void run() {
    tid = threadIdx.x;
    lane = tid & 63;
    g = lane >> 4;
    n = lane & 15;
    wave = wave_uniform(tid >> 6);
    const int lb = xcd_major_block((int)blockIdx.x, (int)gridDim.x);
    bh = lb / p.n_qblocks;
    const int qb = lb - bh * p.n_qblocks;
    L = p.L;
    const size_t head_off = (size_t)bh * (size_t)L * D;
    const T* __restrict__ qg = reinterpret_cast<const T*>(p.q) + head_off;
    kg = reinterpret_cast<const T*>(p.k) + head_off;
    vtg = reinterpret_cast<const T*>(p.vt) + (size_t)bh * C::VROWS * p.L_pad;

    row0 = qb * C::ROWS + 16 * TPW * wave;
    const bool act0 = row0 < L, act1 = TPW == 2 && row0 + 16 < L;
    const bool same_row = p.M >= 32;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int r = row0 + 16 * t;
      const int mrow = r < L ? r / p.M : 0;
      mask_row[t] = p.mask + ((size_t)bh * p.T_q + (size_t)mrow) * p.words;
      const int rq = r + n < L ? r + n : L - 1;
#pragma unroll
      for (int s = 0; s < C::NSLAB; ++s)
        tile[t].qf[s] = *reinterpret_cast<const u32x4*>(qg + (size_t)rq * D + C::SLAB * s + VEC * g);
      if (r + n >= L)
#pragma unroll
        for (int s = 0; s < C::NSLAB; ++s) tile[t].qf[s] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j <= C::NDB; ++j) tile[t].oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      tile[t].m_run = -INFINITY;
    }

    // All work-groups of an XCD walk the chunks of their head in the same
    // order, so a chunk is fetched into that XCD's L2 once and read there by
    // every work-group near the same time (staggered start chunks measured
    // slower).
    const int n_chunks = (L + KC - 1) / KC;
    auto phys = [](int c) { return c; };
    uint32_t mcur[TPW][C::MW], mnext[TPW][C::MW];
    issue_chunk(phys(0), 0, mcur);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int c = 0; c < n_chunks; ++c) {
      const int buf = c & 1;
      const bool more = c + 1 < n_chunks;
      // buffer buf^1 was last read in iteration c-1, which every wave has left
      if (more) issue_chunk(phys(c + 1), buf ^ 1, mnext);
      if (act0) compute_chunk(phys(c), buf, mcur, same_row, act1);
      __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of chunk c+1 have landed
      __syncthreads();                 // ... and every other wave's
      if (more) {
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
          for (int i = 0; i < C::MW; ++i) mcur[t][i] = mnext[t][i];
      }
    }

    // normalise and store
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int r = row0 + 16 * t + n;
      if (r >= L) continue;
      Tile& tt = tile[t];
      const float l_tot = tt.oacc[C::NDB][0];
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      T* og = reinterpret_cast<T*>(p.o) + head_off + (size_t)r * D;
#pragma unroll
      for (int j = 0; j < C::NDB; ++j) {
        const f32x4 val = tt.oacc[j] * inv;
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
            l_tot > 0.f ? (tt.m_run + __builtin_log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
      }
    }
  }
};

// Packs V [B*H][L][D] into V^T [B*H][D + 1][L_pad]: row d < D holds V[., d]
// for keys < L and zeros up to L_pad; row D holds ones for keys < L and
// zeros after (the softmax denominator is accumulated against it).  One
// work-group per 64 keys of one (b, h): 16-byte coalesced reads of the rows,
// a transpose through LDS, 16-byte coalesced writes of the columns.
template <typename T, int D>
__global__ __launch_bounds__(256) void vt_pack_kernel(const T* __restrict__ v, T* __restrict__ vt,
                                                      int L, int L_pad) {
  constexpr int VEC = ElemTraits<T>::VEC;
  constexpr int CPR = D / VEC;       // 16-byte chunks per V row
  constexpr int TS = D + 2;          // LDS row stride (elements), odd word stride for bf16
  __shared__ T tile[64 * TS];
  // one-dimensional grid (B*H may exceed the y-dimension limit): block
  // (bh, 64-key group) = blockIdx.x / groups, blockIdx.x % groups
  const unsigned groups = (unsigned)(L_pad / 64);
  const int bh = (int)(blockIdx.x / groups);
  const int k0 = (int)(blockIdx.x - (unsigned)bh * groups) * 64;
  const T* src = v + ((size_t)bh * L) * D;
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int r = i / CPR, ch = i % CPR;
    const int key = k0 + r;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (key < L) x = *reinterpret_cast<const u32x4*>(src + (size_t)key * D + ch * VEC);
    const T* xe = reinterpret_cast<const T*>(&x);
#pragma unroll
    for (int e = 0; e < VEC; ++e) tile[r * TS + ch * VEC + e] = xe[e];
  }
  __syncthreads();
  constexpr int GPR = 64 / VEC;      // 16-byte groups per output row segment
  T* dst = vt + (size_t)bh * (D + 1) * L_pad + k0;
  for (int i = threadIdx.x; i < (D + 1) * GPR; i += 256) {
    const int d = i / GPR, kg = i % GPR;
    T out[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int r = kg * VEC + e;
      if (d < D) {
        out[e] = tile[r * TS + d];
      } else {
        if constexpr (sizeof(T) == 2) out[e] = (T)(k0 + r < L ? 0x3f80u : 0u);
        else out[e] = k0 + r < L ? 1.f : 0.f;
      }
    }
    *reinterpret_cast<u32x4*>(dst + (size_t)d * L_pad + kg * VEC) = *reinterpret_cast<const u32x4*>(out);
  }
}

template <typename T, int D, int N, int KC, int W, int TPW>
__global__ __launch_bounds__(64 * W) void attn_fwd_kernel(AttnParams p) {
  using K = AttnKernel<T, D, N, KC, W, TPW>;
  __shared__ __attribute__((aligned(16))) typename K::Smem sm;
  K k(p, sm);
  k.run();
}

}  // namespace tsa
