// Tile-sparse attention forward kernel for bf16 and key tiles of N >= 8 keys
// (gfx950, wave64, 16x16x32 bf16 MFMA).
//
// Operation: FG-Attn ("FG-Attn: Leveraging Fine-Grained Sparse Attention in
// Video Diffusion Models", section Abstract): the query-key dot products of
// every M x N tile whose keep bit is 0 are skipped and those scores take no
// part in the softmax; O = softmax(scale * Q K^T over kept tiles) V.
//
// With N >= 8 every kept key tile is a whole number of "octets", runs of
// eight consecutive keys starting at a multiple of 8.  The kernel packs kept
// octets, four per pass, into the 32-key contraction of the matrix cores:
//   * A work-group owns 256 consecutive query rows of one (b, h); each of its
//     16 waves owns one 16-row query tile (inside one mask row, M being a
//     multiple of 16) and keeps that tile's Q fragment, O^T accumulator and
//     running max in registers.
//   * Keys stream through LDS in chunks of 128 (K rows, and the V^T columns
//     of the packed V^T workspace), double-buffered, filled by direct
//     global-to-LDS loads issued by all waves; each chunk crosses from L2
//     once per 256 query rows.
//   * Per chunk a wave turns the mask bits of its row into the ascending list
//     of kept octets, one nibble per entry in a 64-bit scalar register, with
//     two lookups in a byte-to-nibble-list table.  A pass takes list entries
//     4p..4p+3; a list shorter than a multiple of four is padded with the
//     first kept octet (real kept scores, so the running max only sees real
//     kept scores), whose probabilities the pass sets to zero.
//   * Scores are formed transposed, S^T = K Q^T (A = K rows from LDS, B = the
//     Q fragment); a 16-key score block holds two whole octets.  The
//     accumulators are directly the B operand of O^T += V^T P^T
//     (probabilities never leave registers); the matching A operand is two
//     8-byte LDS reads of V^T columns per lane.  Row strides are chosen so
//     that both reads are free of LDS bank conflicts for any octets.
//   * The softmax denominator l comes from the same MFMA pipeline, with a
//     constant all-ones A operand in registers.
//   * A chunk's last pass with one or two real octets (the rest padding)
//     forms one score block and runs PV on the 16-key 16x16x16 step, whose
//     operands are that block's probabilities and the first V^T read of
//     each d block: half the V^T reads and exponentials of a full pass, for
//     the same matrix-core time.
//   * Online softmax in base 2 with c = |scale| * log2(e) (a negative scale
//     negates the Q fragment, which is exact).  Every score accumulator
//     starts from -m/c, m the running reference max, so a probability costs
//     one multiply and one exp2 and the block maximum is compared with the
//     rescale threshold as it comes out of the MFMAs.  The reference max is
//     raised (and O, l rescaled) only when some score exceeds it by more than
//     2^8, decided by one wave-wide ballot; the first pass sets it to that
//     pass's maximum.
//   * Keys past L in the last octet read K row L-1 (the loads clamp the row)
//     and zero V^T columns; their probabilities are set to zero.
#pragma once

#include <type_traits>

#include "attention_fwd_impl.h"
#include "launch.h"

namespace tsa {

template <int D, int N, bool F8 = false>
struct OctCfg {
  static constexpr int KC = 128;                   // keys per chunk
  static constexpr int W = 16;                     // waves per work-group
  static constexpr int ROWS = 16 * W;              // query rows per work-group
  static constexpr int OPC = KC / 8;               // octets per chunk
  static constexpr int TPC = KC / N;               // key tiles per chunk (<= 16)
  static constexpr int LOG2R = ilog2(N / 8);       // octets per key tile, log2
  // Q/K elements: bf16, or FP8 (e4m3) whose 16x16x128 matrix-core step
  // takes a whole 128-wide d range: then the Q fragment is two 16-byte halves
  static constexpr int ESZ = F8 ? 1 : 2;           // bytes per Q / K element
  static constexpr int NSLAB = F8 ? 2 : D / 32;    // 32-wide d slabs of the QK^T contraction
  static constexpr int NDB = D / 16;               // 16-wide d blocks of O^T
  static constexpr int KRB = D * ESZ;              // K row bytes in memory
  // K row stride in LDS: with 32 padding bytes, the 16 key rows of a score
  // block (two octets, eight consecutive rows each) read 16 bytes per lane
  // without bank conflicts whatever the octets; V^T rows take 16 padding
  // bytes, which keeps their 8-byte column reads conflict-free.
  static constexpr int KRS = KRB + 32;
  static constexpr int VRB = KC * 2;               // V^T row bytes of one chunk
  static constexpr int VRS = VRB + 16;             // V^T row stride in LDS
  static constexpr int VROWS = D + 1;              // V^T workspace rows (d = 0..D-1, ones row)
  static constexpr int VROWS_LDS = D;              // V^T rows staged (the ones row is not read)
  static constexpr int NI_K = (KC * KRS + 1023) / 1024;     // 1-KB loads per K chunk
  static constexpr int NI_V = (VROWS_LDS * VRS + 1023) / 1024;  // 1-KB loads per V^T chunk
  static constexpr int NK_W = (NI_K + W - 1) / W;                // K pieces per wave
  static constexpr int NV_W = (NI_V + W - 1) / W;                // V^T pieces per wave
  static_assert(N >= 8 && N <= 64 && (N & (N - 1)) == 0, "octet kernel: N in {8,16,32,64}");
  static_assert(D % 32 == 0, "head dim");
  static_assert(!F8 || D == 128, "FP8 scores: d = 128 (one 16x16x128 step)");
  static_assert(TPC <= 16, "tile bits of a chunk fit one mask word");
};

// Entry b (0..255): the set bits of byte b in ascending order, one nibble
// each; entry 256 + b: the same list with 8 added to every entry, for the
// upper byte of a 16-octet mask.
struct OctetNibbleTable {
  uint32_t v[512];
};
constexpr OctetNibbleTable make_octet_nibbles() {
  OctetNibbleTable t{};
  for (int half = 0; half < 2; ++half)
    for (int b = 0; b < 256; ++b) {
      uint32_t x = 0u;
      int j = 0;
      for (int i = 0; i < 8; ++i)
        if ((b >> i) & 1) x |= (uint32_t)(i + 8 * half) << (4 * j++);
      t.v[256 * half + b] = x;
    }
  return t;
}
static __constant__ OctetNibbleTable kOctetNibbles = make_octet_nibbles();

// Octet mask of a chunk from its tile bits (2^LOG2R octets per tile): bit t
// of tb becomes bits t*R .. t*R+R-1 (R = 2^LOG2R).
template <int LOG2R>
__device__ __forceinline__ uint32_t octet_mask(uint32_t tb) {
  if constexpr (LOG2R == 0) {
    return tb;
  } else if constexpr (LOG2R == 1) {
    uint32_t x = (tb | (tb << 4)) & 0x0F0Fu;
    x = (x | (x << 2)) & 0x3333u;
    x = (x | (x << 1)) & 0x5555u;
    return x | (x << 1);
  } else if constexpr (LOG2R == 2) {
    uint32_t x = (tb | (tb << 6)) & 0x0303u;
    x = (x | (x << 3)) & 0x1111u;
    return x * 15u;
  } else {
    return ((tb & 1u) | ((tb & 2u) << 7)) * 255u;
  }
}

// SKIP: the work-group visits only the chunks its bitmap marks as needed
// (work-groups flagged by chunk_need_kernel); otherwise every chunk (the
// work-groups not flagged).
template <int D, int N, bool SKIP, bool F8 = false>
struct OctKernel {
  using C = OctCfg<D, N, F8>;
  static constexpr float RESCALE_STEP = 8.f;  // log2 units the max may grow before rescaling

  struct SmemPlain {
    __attribute__((aligned(16))) uint8_t k[2][C::NI_K * 1024];
    __attribute__((aligned(16))) uint8_t vt[2][C::NI_V * 1024];
  };
  struct SmemSkip : SmemPlain {
    uint16_t clist[kMaxChunks];  // needed chunks, ascending
  };
  using Smem = typename std::conditional<SKIP, SmemSkip, SmemPlain>::type;

  const AttnParams& p;
  Smem& sm;
  int lane, g, n, wave, L;
  const uint8_t* __restrict__ kg;   // K rows of this (b, h), bytes
  const bf16_t* __restrict__ vtg;
  const uint32_t* __restrict__ mrow;
  u32x4 qf[C::NSLAB];
  f32x4 oacc[C::NDB + 1];
  float m_ref;        // reference max of this lane's query (log2 units)
  f32x4 nm4;          // -m_ref / cs in every element: the initial score accumulator
  u32x4 ones;         // bf16 ones: the A operand that sums probabilities into l
  float cs;           // |scale| * log2(e)
  float thr;          // rescale threshold on unscaled scores: -inf before the first pass,
                      // then RESCALE_STEP / cs
  uint32_t doffk[C::NK_W], doffv[C::NV_W];  // per-lane load offsets of a full chunk's K and V^T pieces

  __device__ __forceinline__ OctKernel(const AttnParams& pp, Smem& s) : p(pp), sm(s) {}

  // Byte offset read by lane `ln` for 1-KB load `I` of a chunk with `rows`
  // keys, relative to the chunk's resource base; out of range (reads zero)
  // for the padding bytes of an LDS row.  K rows past the last key repeat it.
  __device__ __forceinline__ uint32_t dma_offset(int I, int ln, int rows) const {
    constexpr uint32_t OOB = 0x80000000u;
    if (I < C::NI_K) {
      const int pos = I * 1024 + 16 * ln;
      const int row = pos / C::KRS, cb = pos - row * C::KRS;
      const int r = row < rows ? row : rows - 1;
      return row < C::KC && cb < C::KRB ? (uint32_t)(r * C::KRB + cb) : OOB;
    }
    const int pos = (I - C::NI_K) * 1024 + 16 * ln;
    const int row = pos / C::VRS, cb = pos - row * C::VRS;
    return row < C::VROWS_LDS && cb < C::VRB ? (uint32_t)(row * p.L_pad * 2 + cb) : OOB;
  }

  // This wave's share of the loads of chunk c into buffer `buf`, and the
  // mask word of chunk c.  Nothing waits here.
  __device__ __forceinline__ uint32_t issue_chunk(int c, int buf) {
    const int kbase = c * C::KC;
    const int rows = L - kbase < C::KC ? L - kbase : C::KC;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kg + (size_t)kbase * C::KRB), (short)0, rows * C::KRB, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vtg + kbase), (short)0, (C::VROWS * p.L_pad - kbase) * 2, kBufferFlags);
    if (rows < C::KC) {  // the last chunk (visited last): K offsets for its rows
#pragma unroll
      for (int u = 0; u < C::NK_W; ++u) {
        const int j = wave + C::W * u;
        if (j < C::NI_K) doffk[u] = dma_offset(j, lane, rows);
      }
    }
    // wave w loads K pieces w, w + W, ... and V^T pieces w, w + W, ...
    typedef __attribute__((address_space(3))) uint8_t* dst_t;
    load_pieces<C::NI_K, C::W>(rk, (dst_t)sm.k[buf], doffk, wave);
    load_pieces<C::NI_V, C::W>(rv, (dst_t)sm.vt[buf], doffv, wave);
    const int wi = (c * C::TPC) >> 5;
    // a scalar load (the mask is read-only here): it does not queue behind
    // the chunk's LDS loads
    return ((const __attribute__((address_space(4))) uint32_t*)mrow)[wi < p.words ? wi : p.words - 1];
  }

  // One pass over the four list positions q0..q0+3 (rem = entries left from
  // q0; positions >= rem are padding).  Score block b (0, 1) holds the octets
  // at positions q0+2b and q0+2b+1, eight key rows each: lane (g, n) reads
  // row n&7 of the octet at position q0+2b+(n>>3), at LDS address ka<b>.
  // The score accumulators leave lane group g with keys 4(g&1)..4(g&1)+3 of
  // octet ovx (position q0+(g>>1)) and of octet ovy (position q0+2+(g>>1)),
  // so its PV operand is two 8-byte V^T reads.  lim: keys of the chunk that
  // exist.  SINGLE (rem <= 2: positions 2 and 3 are padding): one score
  // block, and PV on the 16-key 16x16x16 matrix-core step, whose A operand
  // (keys 4g..4g+3 of the block for lane group g) is the ovx read alone and
  // whose B operand is block 0's probabilities: half the V^T reads and half
  // the exponentials, for the same matrix-core time.
  template <bool SINGLE>
  __device__ __forceinline__ void pass(int buf, uint32_t ka0, uint32_t ka1, int ovx, int ovy, int rem,
                                            int lim) {
    // keeps the ones operand in registers instead of rebuilding it per pass
    asm volatile("" : "+v"(ones));
    f32x4 s0 = nm4, s1 = nm4;
    // Raised wave priority from the score MFMAs through the softmax: a wave
    // that reaches its score block is preferred over waves in their PV
    // phase, which spreads the waves of a SIMD over the phases of a pass.
    __builtin_amdgcn_s_setprio(1);
    if constexpr (F8) {
      // one 16x16x128 FP8 step per score block: 32 bytes of the K row per lane
      if constexpr (SINGLE) {
        s0 = mac_fp8(lds_load<u32x4>(ka0), lds_load<u32x4>(ka0 + 16), qf[0], qf[1], s0);
      } else {
        const u32x4 a0 = lds_load<u32x4>(ka0), a1 = lds_load<u32x4>(ka0 + 16);
        const u32x4 b0 = lds_load<u32x4>(ka1), b1 = lds_load<u32x4>(ka1 + 16);
        s0 = mac_fp8(a0, a1, qf[0], qf[1], s0);
        s1 = mac_fp8(b0, b1, qf[0], qf[1], s1);
      }
    } else if constexpr (SINGLE) {
#pragma unroll
      for (int sl = 0; sl < C::NSLAB; ++sl)
        s0 = Mma<bf16_t>::mac8(lds_load<u32x4>(ka0 + 64 * sl), qf[sl], s0);
    } else {
#pragma unroll
      for (int sl = 0; sl < C::NSLAB; ++sl) {
        const u32x4 a0 = lds_load<u32x4>(ka0 + 64 * sl);
        const u32x4 a1 = lds_load<u32x4>(ka1 + 64 * sl);
        s0 = Mma<bf16_t>::mac8(a0, qf[sl], s0);
        s1 = Mma<bf16_t>::mac8(a1, qf[sl], s1);
      }
    }
    // The first V^T operands are read before the softmax so their latency
    // overlaps it; the rest after, within the register budget.
    constexpr int EARLY = C::NDB / 2 - 1;
    const int half = 8 * (g & 1);
    const uint32_t vb = lds_addr(sm.vt[buf]) + (uint32_t)(n * C::VRS + half);
    const uint32_t vx = shl4_add((uint32_t)ovx, vb);
    const uint32_t vy = shl4_add((uint32_t)ovy, vb);
    u32x4 av[C::NDB];
    u32x2 ax[C::NDB];
    auto vread = [&](int j) {
      if constexpr (SINGLE) {
        ax[j] = lds_load<u32x2>(vx + 16 * j * C::VRS);
      } else {
        const u32x2 x = lds_load<u32x2>(vx + 16 * j * C::VRS);
        const u32x2 y = lds_load<u32x2>(vy + 16 * j * C::VRS);
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
    // (built with NaNs assumed absent, these fold into three-way max
    // instructions without operand quieting)
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
    s0 *= cs;
    if constexpr (!SINGLE) s1 *= cs;
    f32x4 e0, e1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e0[i] = exp2_fast(s0[i]);
      if constexpr (!SINGLE) e1[i] = exp2_fast(s1[i]);
    }
    // keys past the end of the sequence (in the last, partial octet) carry no
    // probability
    if (lim & 7) {
      const int k0 = 8 * ovx + 4 * (g & 1), k1 = 8 * ovy + 4 * (g & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (k0 + i >= lim) e0[i] = 0.f;
        if constexpr (!SINGLE)
          if (k1 + i >= lim) e1[i] = 0.f;
      }
    }
    if constexpr (SINGLE) {
      bf16x4 pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = (__bf16)e0[i];
      u32x2 bop = __builtin_bit_cast(u32x2, pb);
      // position 1 is padding when rem == 1
      if ((g >> 1) >= rem) bop = u32x2{0u, 0u};
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int j = EARLY; j < C::NDB; ++j) vread(j);
      const bf16x4 b4 = __builtin_bit_cast(bf16x4, bop);
#pragma unroll
      for (int j = 0; j < C::NDB; ++j)
        oacc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, ax[j]), b4, oacc[j], 0, 0, 0);
      const u32x2 o2 = u32x2{ones[0], ones[1]};
      oacc[C::NDB] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, o2), b4, oacc[C::NDB], 0, 0, 0);
    } else {
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = (__bf16)e0[i];
        pb[4 + i] = (__bf16)e1[i];
      }
      u32x4 bop = __builtin_bit_cast(u32x4, pb);
      // padding list positions (the last pass of a list) carry no probability
      if (rem < 4) {
        if ((g >> 1) >= rem) { bop[0] = 0u; bop[1] = 0u; }
        if (2 + (g >> 1) >= rem) { bop[2] = 0u; bop[3] = 0u; }
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int j = EARLY; j < C::NDB; ++j) vread(j);
#pragma unroll
      for (int j = 0; j < C::NDB; ++j) oacc[j] = Mma<bf16_t>::mac8(av[j], bop, oacc[j]);
      oacc[C::NDB] = Mma<bf16_t>::mac8(ones, bop, oacc[C::NDB]);
    }
  }

  // kept-octet list of one chunk as a wave-uniform value: entry j (an octet
  // index of the chunk) in bits 4j..4j+3
  struct List {
    uint64_t w;
    int count;
  };

  // Kept octets of chunk c (ascending), padded after the `count` kept
  // entries with the first kept octet (real kept scores, whose probabilities
  // the pass zeroes).  A few scalar instructions and two lookups in a small
  // constant table: no loop, no LDS round trip, and little load on the
  // scalar unit that all waves of a compute unit share.
  __device__ __forceinline__ List make_list(int c, uint32_t mword) const {
    List li{0ull, 0};
    uint32_t tb = uniform_u32(mword) >> ((c * C::TPC) & 31);
    if constexpr (C::TPC < 32) tb &= (1u << C::TPC) - 1u;
    const int left = L - c * C::KC;                   // keys of this chunk that exist
    const int nval = left >= C::KC ? C::OPC : (left + 7) >> 3;
    const uint32_t m = octet_mask<C::LOG2R>(tb) & ((1u << nval) - 1u);
    const uint32_t lo = m & 255u, hi = m >> 8;
    const int clo = __builtin_popcount(lo);
    li.count = clo + __builtin_popcount(hi);
    uint64_t w = (uint64_t)kOctetNibbles.v[lo] | ((uint64_t)kOctetNibbles.v[256 + hi] << (4 * clo));
    if (li.count != 0 && li.count < 16) w |= (0x1111111111111111ull * (w & 15u)) << (4 * li.count);
    li.w = w;
    return li;
  }

  // The passes of one chunk (lim: keys of the chunk that exist): each pass
  // takes the next four list entries as a wave-uniform 16-bit value and every
  // lane extracts the entries it needs.
  __device__ __forceinline__ void run_list(int buf, const List& li, int lim) {
    const uint32_t shq = 4u * (uint32_t)(n >> 3), shv = 4u * (uint32_t)(g >> 1);
    const uint32_t kb = lds_addr(sm.k[buf]) + (uint32_t)((n & 7) * C::KRS + (F8 ? 32 : 16) * g);
    uint64_t rest = li.w;
    int q0 = 0;
    // passes with at least three real octets, then at most one with one or two
    for (; li.count - q0 > 2; q0 += 4) {
      const uint32_t w = (uint32_t)rest & 0xffffu;
      rest >>= 16;
      const uint32_t ka0 = mad_u24(__builtin_amdgcn_ubfe(w, shq, 4), 8u * C::KRS, kb);
      const uint32_t ka1 = mad_u24(__builtin_amdgcn_ubfe(w, shq + 8u, 4), 8u * C::KRS, kb);
      const int ovx = (int)__builtin_amdgcn_ubfe(w, shv, 4);
      const int ovy = (int)__builtin_amdgcn_ubfe(w, shv + 8u, 4);
      pass<false>(buf, ka0, ka1, ovx, ovy, li.count - q0, lim);
    }
    if (q0 < li.count) {
      const uint32_t w = (uint32_t)rest & 0xffffu;
      const uint32_t ka0 = mad_u24(__builtin_amdgcn_ubfe(w, shq, 4), 8u * C::KRS, kb);
      const int ovx = (int)__builtin_amdgcn_ubfe(w, shv, 4);
      pass<true>(buf, ka0, ka0, ovx, ovx, li.count - q0, lim);
    }
  }

  __device__ __forceinline__ void run() {
    const int tid = threadIdx.x;
    lane = tid & 63;
    g = lane >> 4;
    n = lane & 15;
    wave = wave_uniform(tid >> 6);
    const int lb = xcd_major_block((int)blockIdx.x, (int)gridDim.x);
    // The plain and the skipping kernel each run the work-groups of their
    // kind.  Skipping is used only when at least a quarter of all
    // work-groups would gain from it: the skipping kernel runs after the
    // plain one, so a few flagged work-groups would run alone at the end.
    if (p.need_flag != nullptr) {
      // (flag 2: the work-group needs no chunk at all, e.g. a skipped head;
      // the skipping kernel writes its zero rows without staging anything)
      const bool many = (long long)wave_uniform((int)*p.need_count) * 4 >= (long long)gridDim.x;
      const int f = wave_uniform((int)p.need_flag[lb]);
      const bool mine = f == 2 || (many && f == 1);
      if (mine != SKIP) return;
    } else if (SKIP) {
      return;
    }
    const int bh = lb / p.n_qblocks;
    const int qb = lb - bh * p.n_qblocks;
    L = p.L;
    const size_t head_off = (size_t)bh * (size_t)L * D;
    kg = reinterpret_cast<const uint8_t*>(p.k) + head_off * C::ESZ;
    vtg = reinterpret_cast<const bf16_t*>(p.vt) + (size_t)bh * C::VROWS * p.L_pad;

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
    if (cs < 0.f) {  // c * s = |c| * ((-q) . k), and negating bf16 / FP8 is exact
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
    // The fragment is complete here: later code sees registers written by
    // this statement, not loads in flight, so no load wait lands in the
    // chunk loop.
#pragma unroll
    for (int s = 0; s < C::NSLAB; ++s) asm volatile("" : "+v"(qf[s]));
#pragma unroll
    for (int j = 0; j <= C::NDB; ++j) oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref = 0.f;
    nm4 = f32x4{0.f, 0.f, 0.f, 0.f};
    thr = -INFINITY;
    ones = u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};

#pragma unroll
    for (int u = 0; u < C::NK_W; ++u) {
      const int j = wave + C::W * u;
      doffk[u] = j < C::NI_K ? dma_offset(j, lane, C::KC) : 0u;
    }
#pragma unroll
    for (int u = 0; u < C::NV_W; ++u) {
      const int j = wave + C::W * u;
      doffv[u] = j < C::NI_V ? dma_offset(C::NI_K + j, lane, C::KC) : 0u;
    }
    const int n_chunks = (L + C::KC - 1) / C::KC;
    if constexpr (SKIP) {
      // The needed chunks, ascending, into an LDS list: lane i of wave 0
      // expands bitmap word i at its prefix-sum offset.
      const int nw = (n_chunks + 31) >> 5;
      const uint32_t needv = lane < nw ? p.need[(size_t)lb * kNeedWords + lane] : 0u;
      const int cntw = __builtin_popcount(needv);
      int incl = cntw;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      const int n_need = wave_uniform(__shfl(incl, 63));
      if (wave == 0) {
        int pos = incl - cntw;
        uint32_t bits = needv;
        while (bits != 0u) {
          const int b = __builtin_ctz(bits);
          bits &= bits - 1u;
          sm.clist[pos++] = (uint16_t)(32 * lane + b);
        }
      }
      __syncthreads();
      auto chunk_at = [&](int k) -> int {
        return k < n_need ? (int)uniform_u32(sm.clist[k]) : n_chunks;
      };
      int k = 0;
      int c = chunk_at(0);
      List cur = {0ull, 0};
      if (c < n_chunks) {
        const uint32_t m0 = issue_chunk(c, 0);
        __builtin_amdgcn_s_waitcnt(0);
        if (act) cur = make_list(c, m0);
      }
      int cn = chunk_at(1);
      __syncthreads();
      for (int buf = 0; c < n_chunks; buf ^= 1) {
        const bool more = cn < n_chunks;
        // buffer buf^1 was last read in the previous iteration, which every
        // wave has left
        const uint32_t mnext = more ? issue_chunk(cn, buf ^ 1) : 0u;
        const int cnn = chunk_at(k + 2);
        if (act) run_list(buf, cur, L - c * C::KC < C::KC ? L - c * C::KC : C::KC);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk cn have landed
        if (act && more) cur = make_list(cn, mnext);
        __syncthreads();                // ... and every other wave's
        c = cn;
        cn = cnn;
        ++k;
      }
    } else {
      const uint32_t m0 = issue_chunk(0, 0);
      __builtin_amdgcn_s_waitcnt(0);
      List cur = {0ull, 0};
      if (act) cur = make_list(0, m0);
      __syncthreads();
      for (int c = 0; c < n_chunks; ++c) {
        const int buf = c & 1;
        const bool more = c + 1 < n_chunks;
        // buffer buf^1 was last read in iteration c-1, which every wave has left
        const uint32_t mnext = more ? issue_chunk(c + 1, buf ^ 1) : 0u;
        if (act) run_list(buf, cur, L - c * C::KC < C::KC ? L - c * C::KC : C::KC);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk c+1 have landed
        if (act && more) cur = make_list(c + 1, mnext);
        __syncthreads();                // ... and every other wave's
      }
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

template <int D, int N, bool SKIP, bool F8 = false>
__global__ __launch_bounds__(1024) void attn_oct_kernel(AttnParams p) {
  static_assert(OctCfg<D, N, F8>::W == 16, "launch bounds: 16 waves");
  static_assert(OctCfg<D, N, F8>::KC == kChunkKeys && OctCfg<D, N, F8>::ROWS == kRowsPerGroup, "chunk layout");
  using K = OctKernel<D, N, SKIP, F8>;
  __shared__ __attribute__((aligned(16))) typename K::Smem sm;
  K k(p, sm);
  k.run();
}

// One work-group per attention work-group (logical numbering): ORs the mask
// rows of its 256 query rows word by word, marks the 128-key chunks with a
// kept tile in a bitmap (need, kNeedWords words per work-group) and flags
// the work-group when fewer than 7/8 of the chunks are needed (flag 1, or 2
// when none is; counted in `count`, zeroed beforehand).  Mask padding bits
// past T_k can only mark the last chunk.
template <typename T>
__global__ __launch_bounds__(64) void zero_word_kernel(T* w) {
  if (threadIdx.x == 0) *w = T(0);
}

template <int N>
__global__ __launch_bounds__(256) void chunk_need_kernel(AttnParams p, uint32_t* need, uint32_t* flag,
                                                         uint32_t* count) {
  constexpr int TPC = kChunkKeys / N;  // key tiles per chunk (<= 16)
  constexpr int CPW = 32 / TPC;        // chunks per mask word
  constexpr uint32_t TMASK = (1u << TPC) - 1u;
  __shared__ uint32_t words[kNeedWords];
  __shared__ int cnt;
  const int tid = threadIdx.x;
  const int g = blockIdx.x;
  const int bh = g / p.n_qblocks, qb = g - (g / p.n_qblocks) * p.n_qblocks;
  const int n_chunks = (p.L + kChunkKeys - 1) / kChunkKeys;
  const int nw = (n_chunks + 31) >> 5;
  for (int i = tid; i < kNeedWords; i += 256) words[i] = 0u;
  if (tid == 0) cnt = 0;
  __syncthreads();
  const int r0 = qb * kRowsPerGroup;
  const int r1 = r0 + kRowsPerGroup < p.L ? r0 + kRowsPerGroup : p.L;
  const int i0 = r0 / p.M, i1 = (r1 - 1) / p.M;
  const uint32_t* rows = p.mask + ((size_t)bh * p.T_q + i0) * p.words;
  for (int j = tid; j < p.words; j += 256) {
    uint32_t w = 0u;
    for (int i = 0; i <= i1 - i0; ++i) w |= rows[(size_t)i * p.words + j];
#pragma unroll
    for (int h = 0; h < CPW; ++h) {
      const int c = j * CPW + h;
      if (((w >> (h * TPC)) & TMASK) != 0u && c < n_chunks) atomicOr(&words[c >> 5], 1u << (c & 31));
    }
  }
  __syncthreads();
  if (tid < kNeedWords) {
    need[(size_t)g * kNeedWords + tid] = words[tid];
    if (tid < nw) atomicAdd(&cnt, __builtin_popcount(words[tid]));
  }
  __syncthreads();
  if (tid == 0) {
    const bool f = cnt * 8 < n_chunks * 7;
    flag[g] = cnt == 0 ? 2u : f ? 1u : 0u;
    if (f) atomicAdd(count, 1u);
  }
}

}  // namespace tsa
