// Tile-sparse attention forward kernel for bf16 and key tiles of N < 8 keys
// (gfx950, wave64, 16x16x32 bf16 MFMA).
//
// Operation: FG-Attn ("FG-Attn: Leveraging Fine-Grained Sparse Attention in
// Video Diffusion Models", section Abstract): the query-key dot products of
// every M x N tile whose keep bit is 0 are skipped and those scores take no
// part in the softmax; O = softmax(scale * Q K^T over kept tiles) V.  With
// N = 1 a tile is a single key column of an M-row query tile.
//
// Kept keys are packed one by one, 32 per pass, into the contraction of the
// matrix cores:
//   * Work-groups, waves, chunk staging and the online softmax are those of
//     the octet kernel (N >= 8): 16 waves own 16-row query tiles of 256
//     consecutive rows; keys stream through LDS in double-buffered chunks of
//     128, K and V both as rows (V is not transposed).
//   * Per chunk a wave writes the ascending list of its kept keys (one byte
//     each) into a small LDS area of its own, followed by 32 copies of the
//     first kept key as padding.  Pass p takes list positions 32p..32p+31.
//   * Scores S^T = K Q^T: score block b holds positions 16b..16b+15, lane
//     (g, n) reading 16 bytes of the K row of position 16b+n.
//   * PV: the A operand (V^T, 16 d values x 32 keys) comes from transposing
//     LDS reads of V rows: in each 16-lane group g, lane s points at 4 d
//     values of the key at position 4g+(s>>2), and the read hands lane n the
//     value at d = n of the group's four keys, which is exactly the key order
//     of the S^T accumulators (rows 4g..4g+3 of each score block).
//   * l comes from a register ones operand; probabilities of padding
//     positions and of keys past L are set to zero.
//   * A chunk's last pass with at most 16 real positions forms one score
//     block and runs PV on the 16-key 16x16x16 step (half the V reads and
//     exponentials, the same matrix-core time); at 16 x 1 tiles and 80%
//     sparsity that is the second pass a wave needs in about one chunk in
//     twelve, the one the chunk barrier waits for.
//   * Mask words are read with scalar loads, so they sit in scalar registers
//     and do not queue behind the chunk's LDS loads.
// LDS bank conflicts: K and V rows are 288 bytes apart (160 for d = 64), so
// eight keys read together are conflict-free when their indices differ
// modulo 8; kept keys are arbitrary, so some reads take two or three rounds.
#pragma once

#include "attention_fwd_impl.h"

namespace tsa {

template <int D, int N, bool F8 = false>
struct KeyCfg {
  static constexpr int KC = 128;                   // keys per chunk
  static constexpr int W = 16;                     // waves per work-group
  static constexpr int ROWS = 16 * W;              // query rows per work-group
  static constexpr int TPC = KC / N;               // key tiles per chunk (32, 64, 128)
  static constexpr int MW = TPC / 32;              // mask words per chunk
  static constexpr int LOG2N = ilog2(N);
  // Q/K elements: bf16, or FP8 (e4m3) whose 16x16x128 matrix-core step takes
  // the whole d range: then the Q fragment is two 16-byte halves
  static constexpr int ESZ = F8 ? 1 : 2;           // bytes per Q / K element
  static constexpr int NSLAB = F8 ? 2 : D / 32;    // 32-wide d slabs of the QK^T contraction
  static constexpr int NDB = D / 16;               // 16-wide d blocks of O^T
  // LDS row strides: 32 padding bytes per row for bf16; 16 for FP8 scores,
  // where the smaller chunk (55 KB instead of 57) ran 3% faster at 16 x 1
  // tiles with identical results (bf16 gains nothing from it)
  static constexpr int PAD = F8 ? 16 : 32;
  static constexpr int RB = D * 2;                 // V row bytes in memory
  static constexpr int RS = RB + PAD;              // V row stride in LDS
  static constexpr int KRB = D * ESZ;              // K row bytes in memory
  static constexpr int KRS = KRB + PAD;            // K row stride in LDS
  static constexpr int NI_T = (KC * RS + 1023) / 1024;   // 1-KB loads per V tile
  static constexpr int NI_K = (KC * KRS + 1023) / 1024;  // 1-KB loads per K tile
  static constexpr int NK_W = (NI_T + W - 1) / W;  // V (and bf16 K) pieces per wave
  static constexpr int NKK_W = (NI_K + W - 1) / W; // K pieces per wave
  static constexpr int LIST = KC + 32;             // list bytes per wave (entries + padding)
  static_assert(N == 1 || N == 2 || N == 4, "key kernel: N in {1,2,4}");
  static_assert(D % 32 == 0 && MW >= 1 && MW <= 4, "shape");
  static_assert(!F8 || D == 128, "FP8 scores: d = 128 (one 16x16x128 step)");
  // bf16 K pieces are loaded with the V pieces' offsets and count
  static_assert(F8 || (KRS == RS && NI_K == NI_T), "bf16 K and V tiles share one load geometry");
};

template <int D, int N, bool F8 = false>
struct KeyKernel {
  using C = KeyCfg<D, N, F8>;
  static constexpr float RESCALE_STEP = 8.f;  // log2 units the max may grow before rescaling

  // one staging buffer (K and V rows of a chunk; the two buffers are separate
  // __shared__ objects, see lds_cptr) and the per-wave key lists
  struct Buf {
    __attribute__((aligned(16))) uint8_t k[C::NI_K * 1024];
    __attribute__((aligned(16))) uint8_t v[C::NI_T * 1024];
  };
  struct Lists {
    __attribute__((aligned(16))) uint8_t list[C::W][C::LIST];
  };

  const AttnParams& p;
  Buf& bf0;
  Buf& bf1;
  Lists& ls;
  int lane, g, n, wave, L;
  const uint8_t* __restrict__ kg;
  const bf16_t* __restrict__ vg;
  const uint32_t* __restrict__ mrow;
  uint32_t koff[C::NK_W];  // per-lane offsets of this wave's pieces of a full chunk (V, and bf16 K)
  uint32_t kkoff[F8 ? C::NKK_W : 1];  // the same for FP8 K rows
  u32x4 qf[C::NSLAB];
  f32x4 oacc[C::NDB + 1];
  float m_ref;        // reference max of this lane's query (log2 units)
  f32x4 nm4;          // -m_ref / cs in every element: the initial score accumulator
  u32x4 ones;         // bf16 ones: the A operand that sums probabilities into l
  float cs;           // |scale| * log2(e)
  float thr;          // rescale threshold on unscaled scores: -inf before the first pass,
                      // then RESCALE_STEP / cs

  __device__ __forceinline__ KeyKernel(const AttnParams& pp, Buf& b0, Buf& b1, Lists& l)
      : p(pp), bf0(b0), bf1(b1), ls(l) {}

  template <int B>
  __device__ __forceinline__ Buf& bufr() const {
    return B ? bf1 : bf0;
  }

  // Byte offset read by lane `ln` for 1-KB piece `I` of a chunk's V (or K)
  // tile with `rows` keys, relative to the tile's resource base (LDS rows RS
  // apart, RB bytes each); out of range (reads zero) for the padding bytes of
  // an LDS row.  Rows past the last key repeat it.
  template <int RS = C::RS, int RB = C::RB>
  __device__ __forceinline__ uint32_t dma_offset(int I, int ln, int rows) const {
    constexpr uint32_t OOB = 0x80000000u;
    const int pos = I * 1024 + 16 * ln;
    const int row = pos / RS, cb = pos - row * RS;
    const int r = row < rows ? row : rows - 1;
    return row < C::KC && cb < RB ? (uint32_t)(r * RB + cb) : OOB;
  }

  // This wave's share of the loads of chunk c into buffer `buf`, and the
  // mask words of chunk c (wave-uniform).  Nothing waits here.
  template <int B>
  __device__ __forceinline__ void issue_chunk(int c, uint32_t (&mw)[C::MW]) {
    const int kbase = c * C::KC;
    const int rows = L - kbase < C::KC ? L - kbase : C::KC;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kg + (size_t)kbase * C::KRB), (short)0, rows * C::KRB, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vg + (size_t)kbase * D), (short)0, rows * C::RB, kBufferFlags);
    if (rows < C::KC) {  // the last chunk (issued last): offsets for its rows
#pragma unroll
      for (int u = 0; u < C::NK_W; ++u) {
        const int j = wave + C::W * u;
        koff[u] = dma_offset(j < C::NI_T ? j : 0, lane, rows);
      }
      if constexpr (F8) {
#pragma unroll
        for (int u = 0; u < C::NKK_W; ++u) {
          const int j = wave + C::W * u;
          kkoff[u] = dma_offset<C::KRS, C::KRB>(j < C::NI_K ? j : 0, lane, rows);
        }
      }
    }
    // wave w loads K and V pieces w, w + W, ... (bf16: the same offsets)
    typedef __attribute__((address_space(3))) uint8_t* dst_t;
    if constexpr (F8) load_pieces<C::NI_K, C::W>(rk, (dst_t)bufr<B>().k, kkoff, wave);
    else load_pieces<C::NI_T, C::W>(rk, (dst_t)bufr<B>().k, koff, wave);
    load_pieces<C::NI_T, C::W>(rv, (dst_t)bufr<B>().v, koff, wave);
    const int w0 = (c * C::TPC) >> 5;
    // scalar loads (the mask is read-only here): the words land in scalar
    // registers
    const __attribute__((address_space(4))) uint32_t* m4 =
        (const __attribute__((address_space(4))) uint32_t*)mrow;
#pragma unroll
    for (int i = 0; i < C::MW; ++i) {
      const int wi = w0 + i;
      mw[i] = m4[wi < p.words ? wi : p.words - 1];
    }
  }

  // Kept keys of chunk c, ascending, into this wave's list area, then 32
  // copies of the first kept key; returns the number of kept keys.  Lane l
  // looks at keys l and l+64 of the chunk.  Only mask words are read, so the
  // next chunk's list is written before the chunk barrier.
  __device__ __forceinline__ int make_list(int c, const uint32_t (&mw)[C::MW]) const {
    const int left = L - c * C::KC;  // keys of this chunk that exist
    bool keep[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key = lane + 64 * h;
      const int t = key >> C::LOG2N;  // tile within the chunk
      uint32_t w = uniform_u32(mw[0]);
#pragma unroll
      for (int i = 1; i < C::MW; ++i)
        if ((t >> 5) == i) w = uniform_u32(mw[i]);
      keep[h] = key < left && ((w >> (t & 31)) & 1u);
    }
    const uint64_t b0 = __builtin_amdgcn_ballot_w64(keep[0]);
    const uint64_t b1 = __builtin_amdgcn_ballot_w64(keep[1]);
    const int c0 = __builtin_popcountll(b0);
    const int count = c0 + __builtin_popcountll(b1);
    if (count == 0) return 0;
    uint8_t* lst = ls.list[wave];
    if (keep[0]) lst[prefix_count64(b0)] = (uint8_t)lane;
    if (keep[1]) lst[c0 + prefix_count64(b1)] = (uint8_t)(lane + 64);
    const int first = b0 != 0ull ? __builtin_ctzll(b0) : 64 + __builtin_ctzll(b1);
    if (lane < 32) lst[count + lane] = (uint8_t)first;
    return count;
  }

  // One pass over list positions q0..q0+31 (rem = entries left from q0;
  // positions >= rem are padding).  Score block b holds positions
  // q0+16b..q0+16b+15; the S^T accumulators leave lane group g with the keys
  // at positions q0+4g..q0+4g+3 (block 0) and q0+16+4g.. (block 1), whose V
  // values at d = n two transposing reads per d block deliver.  SINGLE
  // (rem <= 16: positions 16..31 are padding): one score block, and PV on the
  // 16-key 16x16x16 matrix-core step, whose A operand is the block-0 read
  // alone and whose B operand is block 0's four probabilities: half the V
  // reads and half the exponentials, for the same matrix-core time.
  template <int B, bool SINGLE>
  __device__ __forceinline__ void pass(int q0, int rem) {
    // keeps the ones operand in registers instead of rebuilding it per pass
    asm volatile("" : "+v"(ones));
    const uint8_t* lst = ls.list[wave];
    const uint32_t kk0 = lst[q0 + n];
    const int vp = q0 + 4 * g + (n >> 2);
    const uint32_t kv0 = lst[vp];
    const lds_cptr kb = to_lds(bufr<B>().k) + (F8 ? 32 : 16) * g;
    const lds_cptr ka0 = kb + kk0 * C::KRS;
    f32x4 s0 = nm4, s1 = nm4;
    uint32_t kv1 = 0;
    // raised wave priority from the score MFMAs through the softmax (as in
    // the octet kernel)
    __builtin_amdgcn_s_setprio(1);
    if constexpr (F8) {
      // one 16x16x128 FP8 step per score block: lane (g, n) supplies d =
      // 32g..32g+31 of the K row of position q0+16b+n and of its query row
      if constexpr (SINGLE) {
        s0 = mac_fp8(lds_read16(ka0), lds_read16(ka0 + 16), qf[0], qf[1], s0);
      } else {
        const uint32_t kk1 = lst[q0 + 16 + n];
        kv1 = lst[vp + 16];
        const lds_cptr ka1 = kb + kk1 * C::KRS;
        const u32x4 a0 = lds_read16(ka0), a1 = lds_read16(ka0 + 16);
        const u32x4 b0 = lds_read16(ka1), b1 = lds_read16(ka1 + 16);
        s0 = mac_fp8(a0, a1, qf[0], qf[1], s0);
        s1 = mac_fp8(b0, b1, qf[0], qf[1], s1);
      }
    } else if constexpr (SINGLE) {
#pragma unroll
      for (int sl = 0; sl < C::NSLAB; ++sl)
        s0 = Mma<bf16_t>::mac8(lds_read16(ka0 + 64 * sl), qf[sl], s0);
    } else {
      const uint32_t kk1 = lst[q0 + 16 + n];
      kv1 = lst[vp + 16];
      const lds_cptr ka1 = kb + kk1 * C::KRS;
#pragma unroll
      for (int sl = 0; sl < C::NSLAB; ++sl) {
        const u32x4 a0 = lds_read16(ka0 + 64 * sl);
        const u32x4 a1 = lds_read16(ka1 + 64 * sl);
        s0 = Mma<bf16_t>::mac8(a0, qf[sl], s0);
        s1 = Mma<bf16_t>::mac8(a1, qf[sl], s1);
      }
    }
    // V operands: lane (g, n) points at d = 4(n&3)..4(n&3)+3 of its V-side
    // key; the transposing read returns d = n of the group's four keys.
    // EARLY of them are issued before the softmax: none, since every read
    // held across the softmax costs registers the next pass's K reads need
    // (at 16 x 1 and 80% sparsity, two early reads of the 8 d blocks ran
    // 1.6% slower, one 0.6% slower).
    constexpr int EARLY = 0;
    const lds_cptr vb = to_lds(bufr<B>().v) + 8 * (n & 3);
    const lds_cptr va0 = vb + kv0 * C::RS;
    const lds_cptr va1 = vb + kv1 * C::RS;
    // SINGLE: block-0 reads only (ax); else both blocks (av)
    u32x4 av[SINGLE ? 1 : C::NDB];
    u32x2 ax[SINGLE ? C::NDB : 1];
    auto vread = [&](int j) {
      if constexpr (SINGLE) {
        ax[j] = lds_read_tr16(va0 + 32 * j);
      } else {
        const u32x2 x = lds_read_tr16(va0 + 32 * j), y = lds_read_tr16(va1 + 32 * j);
        av[j] = u32x4{x[0], x[1], y[0], y[1]};
      }
    };
#pragma unroll
    for (int j = 0; j < EARLY; ++j) vread(j);
    float mr;
    if constexpr (SINGLE) {
      mr = fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3]));
    } else {
      const float ma = fmaxf(fmaxf(s0[0], s0[1]), s0[2]);
      const float mb = fmaxf(fmaxf(s0[3], s1[0]), s1[1]);
      mr = fmaxf(fmaxf(ma, mb), fmaxf(s1[2], s1[3]));
    }
    if (__builtin_amdgcn_ballot_w64(mr > thr) != 0ull) {
      const float mx = max_across_groups(mr) * cs;
      const float delta = fmaxf(mx, thr == -INFINITY ? -INFINITY : 0.f);
      const float alpha = exp2_fast(fminf(-delta, 0.f));
#pragma unroll
      for (int j = 0; j <= C::NDB; ++j) oacc[j] *= alpha;
      const float ic = cs > 0.f ? 1.f / cs : 0.f;
      thr = cs > 0.f ? RESCALE_STEP * ic : INFINITY;
      m_ref += delta;
      const float nmu = -m_ref * ic;
      nm4 = f32x4{nmu, nmu, nmu, nmu};
      const float du = delta * ic;
      s0 -= du;
      if constexpr (!SINGLE) s1 -= du;
    }
    f32x4 e0, e1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e0[i] = exp2_fast(s0[i] * cs);
      if constexpr (!SINGLE) e1[i] = exp2_fast(s1[i] * cs);
    }
    // padding list positions (the last pass of a list) carry no probability
    if (rem < 32) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * g + i >= rem) e0[i] = 0.f;
        if constexpr (!SINGLE)
          if (16 + 4 * g + i >= rem) e1[i] = 0.f;
      }
    }
    if constexpr (SINGLE) {
      bf16x4 pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = (__bf16)e0[i];
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int j = EARLY; j < C::NDB; ++j) vread(j);
#pragma unroll
      for (int j = 0; j < C::NDB; ++j)
        oacc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, ax[j]), pb, oacc[j], 0, 0, 0);
      oacc[C::NDB] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
          __builtin_bit_cast(bf16x4, u32x2{ones[0], ones[1]}), pb, oacc[C::NDB], 0, 0, 0);
    } else {
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = (__bf16)e0[i];
        pb[4 + i] = (__bf16)e1[i];
      }
      const u32x4 bop = __builtin_bit_cast(u32x4, pb);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int j = EARLY; j < C::NDB; ++j) vread(j);
#pragma unroll
      for (int j = 0; j < C::NDB; ++j) oacc[j] = Mma<bf16_t>::mac8(av[j], bop, oacc[j]);
      oacc[C::NDB] = Mma<bf16_t>::mac8(ones, bop, oacc[C::NDB]);
    }
  }

  // Chunk c from buffer B while chunk c+1 loads into the other buffer.
  template <int B>
  __device__ __forceinline__ void chunk_step(int c, int n_chunks, bool act, int& count) {
    const bool more = c + 1 < n_chunks;
    uint32_t mwn[C::MW];
    // buffer B^1 was last read in the previous step, which every wave has left
    if (more) issue_chunk<B ^ 1>(c + 1, mwn);
    if (act) {
      int q0 = 0;
      for (; count - q0 > 16; q0 += 32) pass<B, false>(q0, count - q0);
      if (q0 < count) pass<B, true>(q0, count - q0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk c+1 have landed
    if (act && more) count = make_list(c + 1, mwn);
    __syncthreads();                // ... and every other wave's
  }

  __device__ __forceinline__ void run() {
    const int tid = threadIdx.x;
    lane = tid & 63;
    g = lane >> 4;
    n = lane & 15;
    wave = wave_uniform(tid >> 6);
    const int lb = xcd_major_block((int)blockIdx.x, (int)gridDim.x);
    const int bh = lb / p.n_qblocks;
    const int qb = lb - bh * p.n_qblocks;
    L = p.L;
    const size_t head_off = (size_t)bh * (size_t)L * D;
    kg = reinterpret_cast<const uint8_t*>(p.k) + head_off * C::ESZ;
    vg = reinterpret_cast<const bf16_t*>(p.v) + head_off;

    const int row0 = qb * C::ROWS + 16 * wave;
    const bool act = row0 < L;
    mrow = p.mask + ((size_t)bh * p.T_q + (size_t)(act ? row0 / p.M : 0)) * p.words;
    const int rq = row0 + n < L ? row0 + n : L - 1;
    // lane (g, n): row n of the tile, d = 8g.. of each 32-wide slab (bf16),
    // or d = 32g..32g+31 (FP8)
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(p.q) + (head_off + (size_t)rq * D) * C::ESZ;
#pragma unroll
    for (int s = 0; s < C::NSLAB; ++s)
      qf[s] = *reinterpret_cast<const u32x4*>(qrow + (F8 ? 32 * g + 16 * s : 64 * s + 16 * g));
    if (row0 + n >= L)
#pragma unroll
      for (int s = 0; s < C::NSLAB; ++s) qf[s] = u32x4{0u, 0u, 0u, 0u};
    cs = p.scale_log2;
    if (cs < 0.f) {  // c*s = |c| * ((-q) . k), and negating bf16 / FP8 is exact
      cs = -cs;
      constexpr uint32_t SIGN = F8 ? 0x80808080u : 0x80008000u;
#pragma unroll
      for (int s = 0; s < C::NSLAB; ++s) qf[s] ^= u32x4{SIGN, SIGN, SIGN, SIGN};
    }
    if constexpr (F8) {
      // scores in FP8 units: the Q tile's and the head's K scale join c
      const int t16 = (L + 15) >> 4;
      cs *= p.q_scale[(size_t)bh * t16 + (act ? row0 >> 4 : 0)] * p.k_scale[bh];
    }
#pragma unroll
    for (int j = 0; j <= C::NDB; ++j) oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref = 0.f;
    nm4 = f32x4{0.f, 0.f, 0.f, 0.f};
    thr = -INFINITY;
    ones = u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};

    const int n_chunks = (L + C::KC - 1) / C::KC;
#pragma unroll
    for (int u = 0; u < C::NK_W; ++u) {
      const int j = wave + C::W * u;
      koff[u] = dma_offset(j < C::NI_T ? j : 0, lane, C::KC);
    }
    if constexpr (F8) {
#pragma unroll
      for (int u = 0; u < C::NKK_W; ++u) {
        const int j = wave + C::W * u;
        kkoff[u] = dma_offset<C::KRS, C::KRB>(j < C::NI_K ? j : 0, lane, C::KC);
      }
    }
    uint32_t mw[C::MW];
    issue_chunk<0>(0, mw);
    __builtin_amdgcn_s_waitcnt(0);
    int count = act ? make_list(0, mw) : 0;
    __syncthreads();
    // two chunks per iteration, so that each step names its buffer statically
    for (int c = 0; c < n_chunks; c += 2) {
      chunk_step<0>(c, n_chunks, act, count);
      if (c + 1 < n_chunks) chunk_step<1>(c + 1, n_chunks, act, count);
    }

    const int r = row0 + n;
    if (r >= L) return;
    const float l_tot = oacc[C::NDB][0];
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16_t* og = reinterpret_cast<bf16_t*>(p.o) + head_off + (size_t)r * D;
#pragma unroll
    for (int j = 0; j < C::NDB; ++j) {
      const f32x4 val = oacc[j] * inv;
      bf16x4 ob;
#pragma unroll
      for (int i = 0; i < 4; ++i) ob[i] = (__bf16)val[i];
      *reinterpret_cast<u32x2*>(og + 16 * j + 4 * g) = __builtin_bit_cast(u32x2, ob);
    }
    if (p.lse != nullptr && g == 0)
      p.lse[(size_t)bh * L + r] =
          l_tot > 0.f ? (m_ref + __builtin_log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
};

template <int D, int N, bool F8 = false>
__global__ __launch_bounds__(1024) void attn_key_kernel(AttnParams p) {
  static_assert(KeyCfg<D, N, F8>::W == 16, "launch bounds: 16 waves");
  using K = KeyKernel<D, N, F8>;
  __shared__ __attribute__((aligned(16))) typename K::Buf b0;
  __shared__ __attribute__((aligned(16))) typename K::Buf b1;
  __shared__ __attribute__((aligned(16))) typename K::Lists lists;
  K k(p, b0, b1, lists);
  k.run();
}

}  // namespace tsa
