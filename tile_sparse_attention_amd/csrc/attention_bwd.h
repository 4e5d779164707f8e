// Tile-sparse attention backward kernels (gfx950, wave64, 16x16x32 bf16 MFMA).
//
// Operation: the gradient, for an upstream gradient dO of the output, of the
// FG-Attn forward ("FG-Attn: Leveraging Fine-Grained Sparse Attention in
// Video Diffusion Models", section Abstract: the scores of every M x N tile
// whose keep bit is 0 are skipped and take no part in the softmax).  The page
// defines only the forward; these are its derivatives.  With P the kept-score
// softmax of the forward, recomputed from the forward's log-sum-exp, and
// D[r] = sum_d dO[r,d] O[r,d] (= sum_c P[r,c] dP[r,c]):
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),
//   dQ = scale dS K,   dK = scale dS^T Q.
// Skipped tiles have P = 0 and cost no matrix-core work.
//
// Three kernels, all on the 16x16 MFMA operand layouts of tsa_device.h:
//   * bwd_prep_kernel: D and lse2 = LSE * log2(e) per row, written per
//     128-row chunk (128 lse2 values, then 128 D values).  A row past L or
//     with no kept key gets lse2 = +inf, which makes its probabilities 0.
//   * bwd_dkdv_kernel: a work-group owns 192 consecutive keys of one (b, h),
//     twelve waves of 16.  Query rows stream through LDS in double-buffered
//     chunks of 128 rows (Q rows, dO rows and the chunk's lse2 / D).  Per
//     chunk each wave lists the 16-row query units in which a tile of one of
//     its keys is kept (M is a multiple of 16, so a unit lies in one mask
//     row) and processes them two at a time:
//       S = Q K_w^T, dP = dO V_w^T   (A = Q / dO rows from LDS, B = the
//                                     wave's K / V fragment in registers),
//       P = 2^(S c - lse2), dS = P (dP - D)   (c = scale log2(e)),
//       dV^T += dO^T P, dK^T += Q^T dS   (A = dO^T / Q^T from transposing
//                                         LDS reads of the same rows).
//     The accumulator layout of S and dP (lane: four query rows of each
//     unit, one key) is directly the B operand of the two updates.
//   * bwd_dq_kernel: a work-group owns 256 query rows (16 waves of 16; 8
//     waves for N = 1 at d = 128), as in the forward; K and V rows stream
//     through LDS in double-buffered
//     chunks of 128 keys.  Per chunk each wave lists its kept keys (one byte
//     each, in LDS) and takes them 32 per pass:
//       S^T = K Q^T, dP^T = V dO^T   (A = K / V rows, B = the wave's Q / dO
//                                     fragments), P^T, dS^T as above,
//       dQ^T += K^T dS^T   (A = K^T from transposing reads of the K rows).
// dK and dV need no atomics (each key belongs to one wave), and dQ is
// recomputed per query instead of accumulated across key blocks.
#pragma once

#include "attention_fwd_octet.h"

namespace tsa {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;      // [B*H][L] natural-log sum-exp from the forward
  const uint32_t* mask;
  void* dq;
  void* dk;
  void* dv;
  float* ld;             // [B*H][n_qc][256]: lse2 of a chunk's 128 rows, then D
  int L, M, T_q, words;
  int n_qc;              // 128-row chunks per (b, h)
  int n_kblocks;         // key blocks per (b, h) (dK/dV grid)
  int n_qblocks;         // 256-row blocks per (b, h) (dQ grid)
  float scale;           // as passed by the caller
  float cs;              // |scale| * log2(e)
};

constexpr int kBwdChunk = 128;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0,
                                           0, 0);
}

// ---------------------------------------------------------------------------
// D = rowsum(dO * O) and lse2 per 128-row chunk: one work-group per chunk
// (block index = (b*H + h) * n_qc + chunk), two threads per row (half a row
// each).
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
  const int bh = (int)blockIdx.x / p.n_qc, c = (int)blockIdx.x - bh * p.n_qc;
  const int t = threadIdx.x, row = t >> 1, half = t & 1;
  const int r = c * kBwdChunk + row;
  float acc = 0.f;
  if (r < p.L) {
    const size_t off = ((size_t)bh * p.L + r) * D + half * (D / 2);
    const u32x4* og = reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(p.o) + off);
    const u32x4* dg = reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(p.dout) + off);
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const u32x4 a = og[i], b = dg[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += __uint_as_float(a[e] << 16) * __uint_as_float(b[e] << 16);
        acc += __uint_as_float(a[e] & 0xffff0000u) * __uint_as_float(b[e] & 0xffff0000u);
      }
    }
  }
  acc += __shfl_xor(acc, 1);
  if (half == 0) {
    float* out = p.ld + ((size_t)bh * p.n_qc + c) * 256;
    float l2 = INFINITY, dd = 0.f;
    if (r < p.L) {
      const float ls = p.lse[(size_t)bh * p.L + r];
      if (ls > -INFINITY && ls < INFINITY) {
        l2 = ls * kLog2e;
        dd = acc;
      }
    }
    out[row] = l2;
    out[kBwdChunk + row] = dd;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: keys owned by waves, query rows streamed.
template <int D>
struct DkdvCfg {
  static constexpr int QC = kBwdChunk;          // query rows per chunk
  static constexpr int UNITS = QC / 16;         // 16-row query units per chunk
  // waves per work-group: 12 (three per SIMD), which leaves each wave the
  // 168 registers its fragments, accumulators and pass need
  static constexpr int W = 12;
  static constexpr int KEYS = 16 * W;           // keys per work-group
  static constexpr int NSLAB = D / 32;          // 32-wide d slabs of S and dP
  static constexpr int NDB = D / 16;            // 16-wide d blocks of dK^T, dV^T
  static constexpr int RB = 2 * D;              // Q / dO row bytes in memory
  static constexpr int RS = RB + 32;            // row stride in LDS
  static constexpr int NI_T = (QC * RS + 1023) / 1024;  // 1-KB loads per Q (or dO) tile
  static constexpr int NQ_W = (NI_T + W - 1) / W;       // Q (and dO) pieces per wave
  static_assert(UNITS == 8 && D % 32 == 0, "shape");
};

template <int D, int N>
struct DkdvKernel {
  using C = DkdvCfg<D>;
  static constexpr int LOG2N = ilog2(N);
  static constexpr int TPW = N >= 16 ? 1 : 16 / N;  // key tiles a wave's 16 keys span

  // one staging buffer; the two buffers are separate __shared__ objects
  struct Buf {
    __attribute__((aligned(16))) uint8_t q[C::NI_T * 1024];
    __attribute__((aligned(16))) uint8_t o[C::NI_T * 1024];  // dO rows
    __attribute__((aligned(16))) float ld[256];               // lse2, then D
  };

  // query units of one chunk with a kept tile for this wave (bit u of
  // `units`, wave-uniform); keep: per lane, bit u = the lane's key is kept
  // (and exists) in unit u
  struct Units {
    uint32_t units;
    uint32_t keep;
  };

  const BwdParams& p;
  Buf& bf0;
  Buf& bf1;
  int lane, g, n, wave, L;
  int mword, tshift;     // mask word and bit of this wave's first key tile
  const bf16_t* __restrict__ qg;
  const bf16_t* __restrict__ og;
  const float* __restrict__ ldg;
  const uint32_t* __restrict__ mhead;
  u32x4 kf[C::NSLAB], vf[C::NSLAB];
  f32x4 dk[C::NDB], dv[C::NDB];
  float cs;
  uint32_t qoff[C::NQ_W];  // per-lane offsets of this wave's Q / dO pieces of a full chunk

  __device__ __forceinline__ DkdvKernel(const BwdParams& pp, Buf& b0, Buf& b1) : p(pp), bf0(b0), bf1(b1) {}

  template <int B>
  __device__ __forceinline__ Buf& bufr() const {
    return B ? bf1 : bf0;
  }

  // Byte offset read by lane `ln` for 1-KB piece I of a chunk's Q (or dO)
  // tile with `rows` query rows; out of range (zero) for row padding; rows
  // past the last repeat it.
  __device__ __forceinline__ uint32_t dma_offset(int I, int ln, int rows) const {
    constexpr uint32_t OOB = 0x80000000u;
    const int pos = I * 1024 + 16 * ln;
    const int row = pos / C::RS, cb = pos - row * C::RS;
    const int r = row < rows ? row : rows - 1;
    return row < C::QC && cb < C::RB ? (uint32_t)(r * C::RB + cb) : OOB;
  }

  // This wave's share of the loads of chunk c into buffer buf, and (lane
  // u < UNITS) the mask word of query unit u; nothing waits here.
  template <int B>
  __device__ __forceinline__ uint32_t issue_chunk(int c) {
    const int q0 = c * C::QC;
    const int rows = L - q0 < C::QC ? L - q0 : C::QC;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(qg + (size_t)q0 * D), (short)0, rows * C::RB, kBufferFlags);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(og + (size_t)q0 * D), (short)0, rows * C::RB, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(ldg + (size_t)c * 256), (short)0, 1024, kBufferFlags);
    if (rows < C::QC) {  // the last chunk (issued last): offsets for its rows
#pragma unroll
      for (int u = 0; u < C::NQ_W; ++u) {
        const int j = wave + C::W * u;
        qoff[u] = dma_offset(j < C::NI_T ? j : 0, lane, rows);
      }
    }
    // wave w loads Q and dO pieces w, w + W, ... (same offsets), wave 0 also
    // the chunk's lse2 / D block
    typedef __attribute__((address_space(3))) uint8_t* dst_t;
    load_pieces<C::NI_T, C::W>(rq, (dst_t)bufr<B>().q, qoff, wave);
    load_pieces<C::NI_T, C::W>(ro, (dst_t)bufr<B>().o, qoff, wave);
    if (wave == 0) dma16(rl, bufr<B>().ld, 16u * (uint32_t)lane);
    const int r = q0 + 16 * (lane & (C::UNITS - 1)) < L ? q0 + 16 * (lane & (C::UNITS - 1)) : L - 1;
    return mhead[(size_t)(r / p.M) * p.words + mword];
  }

  // Units of chunk c from the mask words issue_chunk returned (lane u holds
  // unit u's word): one ballot for the unit set, and per lane the keep bits
  // of its key.
  __device__ __forceinline__ Units make_units(int c, uint32_t mwv, bool kvalid) const {
    const int q0 = c * C::QC;
    const uint32_t f = (mwv >> tshift) & ((1u << TPW) - 1u);
    const bool kept = lane < C::UNITS && q0 + 16 * lane < L && f != 0u;
    Units un{(uint32_t)__builtin_amdgcn_ballot_w64(kept), 0u};
#pragma unroll
    for (int u = 0; u < C::UNITS; ++u) {
      const uint32_t fu = (uint32_t)__builtin_amdgcn_readlane((int)f, u);
      const uint32_t kbit = N >= 16 ? (fu & 1u) : ((fu >> (n >> LOG2N)) & 1u);
      un.keep |= ((un.units >> u) & kbit) << u;
    }
    if (!kvalid) un.keep = 0u;
    return un;
  }

  // Query units u0 and u1 of the chunk in buffer B (single: u1 is padding).
  template <int B>
  __device__ __forceinline__ void pass(int u0, int u1, bool single, uint32_t keep) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, d0 = s0, d1 = s0;
    {
      const lds_cptr qa = to_lds(bufr<B>().q) + 16 * g;
      const lds_cptr oa = to_lds(bufr<B>().o) + 16 * g;
      const uint32_t r0 = (uint32_t)(16 * u0 + n) * C::RS, r1 = (uint32_t)(16 * u1 + n) * C::RS;
#pragma unroll
      for (int sl = 0; sl < C::NSLAB; ++sl) {
        s0 = Mma<bf16_t>::mac8(lds_read16(qa + r0 + 64 * sl), kf[sl], s0);
        d0 = Mma<bf16_t>::mac8(lds_read16(oa + r0 + 64 * sl), vf[sl], d0);
        if (!single) {
          s1 = Mma<bf16_t>::mac8(lds_read16(qa + r1 + 64 * sl), kf[sl], s1);
          d1 = Mma<bf16_t>::mac8(lds_read16(oa + r1 + 64 * sl), vf[sl], d1);
        }
      }
    }
    // lse2 and D of the four query rows each accumulator lane holds
    const float* lb = bufr<B>().ld;
    const f32x4 l0 = *reinterpret_cast<const f32x4*>(lb + 16 * u0 + 4 * g);
    const f32x4 l1 = *reinterpret_cast<const f32x4*>(lb + 16 * u1 + 4 * g);
    const f32x4 e0 = *reinterpret_cast<const f32x4*>(lb + C::QC + 16 * u0 + 4 * g);
    const f32x4 e1 = *reinterpret_cast<const f32x4*>(lb + C::QC + 16 * u1 + 4 * g);
    const bool k0 = (keep >> u0) & 1u;
    const bool k1 = !single && ((keep >> u1) & 1u);
    bf16x8 pb, sb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p0 = k0 ? exp2_fast(__builtin_fmaf(s0[i], cs, -l0[i])) : 0.f;
      const float p1 = k1 ? exp2_fast(__builtin_fmaf(s1[i], cs, -l1[i])) : 0.f;
      pb[i] = (__bf16)p0;
      pb[4 + i] = (__bf16)p1;
      sb[i] = (__bf16)(p0 * (d0[i] - e0[i]));
      sb[4 + i] = (__bf16)(p1 * (d1[i] - e1[i]));
    }
    const u32x4 pbo = __builtin_bit_cast(u32x4, pb), sbo = __builtin_bit_cast(u32x4, sb);
    // transposing reads: lane (g, n) points at row 4g + n/4 of unit u_b,
    // d = 16j + 4(n%4) .. +3; it receives d = 16j + n of rows 4g..4g+3
    const uint32_t tb = (uint32_t)(8 * (n & 3));
    const uint32_t t0 = (uint32_t)(16 * u0 + 4 * g + (n >> 2)) * C::RS + tb;
    const uint32_t t1 = (uint32_t)(16 * u1 + 4 * g + (n >> 2)) * C::RS + tb;
    const lds_cptr qt = to_lds(bufr<B>().q);
    const lds_cptr ot = to_lds(bufr<B>().o);
    auto tr = [&](lds_cptr base, int j) {
      const u32x2 x = lds_read_tr16(base + t0 + 32u * j), y = lds_read_tr16(base + t1 + 32u * j);
      return u32x4{x[0], x[1], y[0], y[1]};
    };
#pragma unroll
    for (int j = 0; j < C::NDB; ++j) {
      dv[j] = Mma<bf16_t>::mac8(tr(ot, j), pbo, dv[j]);
      dk[j] = Mma<bf16_t>::mac8(tr(qt, j), sbo, dk[j]);
    }
  }

  // The chunk's units two at a time (ascending; an odd last one alone);
  // after_first runs after the first pass, or at once when there is none.
  template <int B, typename F>
  __device__ __forceinline__ void run_units(const Units& un, F&& after_first) {
    uint32_t m = un.units;
    auto step = [&] {
      const int u0 = __builtin_ctz(m);
      m &= m - 1u;
      const bool single = m == 0u;
      const int u1 = single ? u0 : __builtin_ctz(m);
      if (!single) m &= m - 1u;
      pass<B>(u0, u1, single, un.keep);
    };
    if (m != 0u) step();
    after_first();
    while (m != 0u) step();
  }

  // Chunk c from buffer B while chunk c+1 loads into the other buffer.  A
  // wave issues its share of chunk c+1's loads after its first pass: issued
  // by every wave at the chunk start, they fill the compute unit's load
  // queue and each wave stalls until its share is accepted, while after one
  // pass the queue drains behind the matrix-core work.
  template <int B>
  __device__ __forceinline__ void chunk_step(int c, int n_chunks, bool act, bool kvalid, Units& cur) {
    const bool more = c + 1 < n_chunks;
    // buffer B^1 was last read in the previous step, which every wave has left
    uint32_t mwn = 0u;
    auto issue = [&] {
      if (more) mwn = issue_chunk<B ^ 1>(c + 1);
    };
    if (act)
      run_units<B>(cur, issue);
    else
      issue();
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk c+1 have landed
    if (act && more) cur = make_units(c + 1, mwn, kvalid);
    __syncthreads();                // ... and every other wave's
  }

  __device__ __forceinline__ void run() {
    const int tid = threadIdx.x;
    lane = tid & 63;
    g = lane >> 4;
    n = lane & 15;
    wave = wave_uniform(tid >> 6);
    const int lb = xcd_major_block((int)blockIdx.x, (int)gridDim.x);
    const int bh = lb / p.n_kblocks;
    const int kb = lb - bh * p.n_kblocks;
    L = p.L;
    const size_t head = (size_t)bh * (size_t)L * D;
    qg = reinterpret_cast<const bf16_t*>(p.q) + head;
    og = reinterpret_cast<const bf16_t*>(p.dout) + head;
    ldg = p.ld + (size_t)bh * p.n_qc * 256;
    mhead = p.mask + (size_t)bh * p.T_q * p.words;
    const int key0 = kb * C::KEYS + 16 * wave;  // first key of this wave
    const bool act = key0 < L;
    const int tile0 = act ? key0 / N : 0;
    mword = tile0 >> 5;
    tshift = tile0 & 31;
    const int key = key0 + n;
    const bool kvalid = key < L;
    const int kr = kvalid ? key : L - 1;
    const bf16_t* kp = reinterpret_cast<const bf16_t*>(p.k) + head + (size_t)kr * D;
    const bf16_t* vp = reinterpret_cast<const bf16_t*>(p.v) + head + (size_t)kr * D;
#pragma unroll
    for (int s = 0; s < C::NSLAB; ++s) {
      kf[s] = *reinterpret_cast<const u32x4*>(kp + 32 * s + 8 * g);
      vf[s] = *reinterpret_cast<const u32x4*>(vp + 32 * s + 8 * g);
    }
    if (!kvalid)
#pragma unroll
      for (int s = 0; s < C::NSLAB; ++s) {
        kf[s] = u32x4{0u, 0u, 0u, 0u};
        vf[s] = u32x4{0u, 0u, 0u, 0u};
      }
    cs = p.cs;
    if (p.scale < 0.f)  // c * s = |c| * (q . (-k)), and negating bf16 is exact
#pragma unroll
      for (int s = 0; s < C::NSLAB; ++s) kf[s] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    // the fragments are complete here: no load wait lands in the chunk loop
#pragma unroll
    for (int s = 0; s < C::NSLAB; ++s) {
      asm volatile("" : "+v"(kf[s]));
      asm volatile("" : "+v"(vf[s]));
    }
#pragma unroll
    for (int j = 0; j < C::NDB; ++j) {
      dk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int n_chunks = p.n_qc;
#pragma unroll
    for (int u = 0; u < C::NQ_W; ++u) {
      const int j = wave + C::W * u;
      qoff[u] = dma_offset(j < C::NI_T ? j : 0, lane, C::QC);
    }
    const uint32_t mw0 = issue_chunk<0>(0);
    __builtin_amdgcn_s_waitcnt(0);
    Units cur{0u, 0u};
    if (act) cur = make_units(0, mw0, kvalid);
    __syncthreads();
    // two chunks per iteration, so that each step names its buffer statically
    for (int c = 0; c < n_chunks; c += 2) {
      chunk_step<0>(c, n_chunks, act, kvalid, cur);
      if (c + 1 < n_chunks) chunk_step<1>(c + 1, n_chunks, act, kvalid, cur);
    }

    if (!kvalid) return;
    bf16_t* dkg = reinterpret_cast<bf16_t*>(p.dk) + head + (size_t)key * D;
    bf16_t* dvg = reinterpret_cast<bf16_t*>(p.dv) + head + (size_t)key * D;
#pragma unroll
    for (int j = 0; j < C::NDB; ++j) {
      bf16x4 a, b;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = (__bf16)(dk[j][i] * p.scale);
        b[i] = (__bf16)dv[j][i];
      }
      *reinterpret_cast<u32x2*>(dkg + 16 * j + 4 * g) = __builtin_bit_cast(u32x2, a);
      *reinterpret_cast<u32x2*>(dvg + 16 * j + 4 * g) = __builtin_bit_cast(u32x2, b);
    }
  }
};

template <int D, int N>
__global__ __launch_bounds__(768) void bwd_dkdv_kernel(BwdParams p) {
  static_assert(DkdvCfg<D>::W == 12, "launch bounds: 12 waves");
  using K = DkdvKernel<D, N>;
  __shared__ __attribute__((aligned(16))) typename K::Buf b0;
  __shared__ __attribute__((aligned(16))) typename K::Buf b1;
  K k(p, b0, b1);
  k.run();
}

// ---------------------------------------------------------------------------
// dQ: query rows owned by waves, keys streamed (per-key lists, any N).
template <int D, int N>
struct DqCfg {
  static constexpr int KC = kBwdChunk;          // keys per chunk
  // waves per work-group: 16 (four per SIMD, 128 registers each), but 8 for
  // N = 1, whose four mask words per chunk do not fit beside the rest
  static constexpr int W = D == 128 && N == 1 ? 8 : 16;
  static constexpr int ROWS = 16 * W;           // query rows per work-group
  static constexpr int NSLAB = D / 32;
  static constexpr int NDB = D / 16;
  static constexpr int RB = 2 * D;              // K / V row bytes in memory
  static constexpr int RS = RB + 32;            // row stride in LDS
  static constexpr int NI_T = (KC * RS + 1023) / 1024;  // 1-KB loads per K (or V) tile
  static constexpr int LIST = KC + 32;          // list bytes per wave (entries + padding)
};

template <int D, int N>
struct DqKernel {
  using C = DqCfg<D, N>;
  static constexpr int LOG2N = ilog2(N);
  static constexpr int TPC = C::KC / N;                 // key tiles per chunk
  static constexpr int MW = TPC >= 32 ? TPC / 32 : 1;   // mask words per chunk

  // one staging buffer (the two are separate __shared__ objects) and the
  // per-wave key lists
  struct Buf {
    __attribute__((aligned(16))) uint8_t k[C::NI_T * 1024];
    __attribute__((aligned(16))) uint8_t v[C::NI_T * 1024];
  };
  struct Lists {
    __attribute__((aligned(16))) uint8_t list[C::W][C::LIST];
  };

  const BwdParams& p;
  Buf& bf0;
  Buf& bf1;
  Lists& ls;
  int lane, g, n, wave, L;
  const bf16_t* __restrict__ kg;
  const bf16_t* __restrict__ vg;
  const uint32_t* __restrict__ mrow;
  u32x4 qf[C::NSLAB], df[C::NSLAB];
  f32x4 dq[C::NDB];
  float l2, dd, cs;  // lse2 and D of this lane's query row
  static constexpr int NK_W = (C::NI_T + C::W - 1) / C::W;  // K (and V) pieces per wave
  uint32_t koff[NK_W];  // per-lane offsets of this wave's pieces of a full chunk

  __device__ __forceinline__ DqKernel(const BwdParams& pp, Buf& b0, Buf& b1, Lists& l)
      : p(pp), bf0(b0), bf1(b1), ls(l) {}

  template <int B>
  __device__ __forceinline__ Buf& bufr() const {
    return B ? bf1 : bf0;
  }

  // Byte offset read by lane `ln` for 1-KB piece I of a chunk's K (or V)
  // tile with `rows` keys; out of range (zero) for row padding; rows past
  // the last repeat it.
  __device__ __forceinline__ uint32_t dma_offset(int I, int ln, int rows) const {
    constexpr uint32_t OOB = 0x80000000u;
    const int pos = I * 1024 + 16 * ln;
    const int row = pos / C::RS, cb = pos - row * C::RS;
    const int r = row < rows ? row : rows - 1;
    return row < C::KC && cb < C::RB ? (uint32_t)(r * C::RB + cb) : OOB;
  }

  template <int B>
  __device__ __forceinline__ void issue_chunk(int c, uint32_t (&mw)[MW]) {
    const int kbase = c * C::KC;
    const int rows = L - kbase < C::KC ? L - kbase : C::KC;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kg + (size_t)kbase * D), (short)0, rows * C::RB, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vg + (size_t)kbase * D), (short)0, rows * C::RB, kBufferFlags);
    if (rows < C::KC) {  // the last chunk (issued last): offsets for its rows
#pragma unroll
      for (int u = 0; u < NK_W; ++u) {
        const int j = wave + C::W * u;
        koff[u] = dma_offset(j < C::NI_T ? j : 0, lane, rows);
      }
    }
    // wave w loads K and V pieces w, w + W, ... (same offsets)
    typedef __attribute__((address_space(3))) uint8_t* dst_t;
    load_pieces<C::NI_T, C::W>(rk, (dst_t)bufr<B>().k, koff, wave);
    load_pieces<C::NI_T, C::W>(rv, (dst_t)bufr<B>().v, koff, wave);
    const int w0 = (c * TPC) >> 5;
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const int wi = w0 + i;
      mw[i] = mrow[wi < p.words ? wi : p.words - 1];
    }
  }

  // Kept keys of chunk c, ascending, into this wave's list area, then 32
  // copies of the first kept key; returns the number of kept keys.  Lane l
  // looks at keys l and l + 64 of the chunk.
  __device__ __forceinline__ int make_list(int c, const uint32_t (&mw)[MW]) const {
    const int left = L - c * C::KC;
    const int bit0 = TPC < 32 ? (c * TPC) & 31 : 0;  // bit of the chunk's first tile
    bool keep[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key = lane + 64 * h;
      const int b = bit0 + (key >> LOG2N);
      uint32_t w = uniform_u32(mw[0]);
#pragma unroll
      for (int i = 1; i < MW; ++i)
        if ((b >> 5) == i) w = uniform_u32(mw[i]);
      keep[h] = key < left && ((w >> (b & 31)) & 1u);
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

  // List positions q0..q0+31 (rem = entries left from q0; positions >= rem
  // are padding).  Score block b holds positions q0+16b..q0+16b+15; the
  // accumulators leave lane group g with positions 4g..4g+3 of each block.
  template <int B>
  __device__ __forceinline__ void pass(int q0, int rem) {
    const bool single = rem <= 16;
    const uint8_t* lst = ls.list[wave];
    const uint32_t kk0 = lst[q0 + n], kk1 = lst[q0 + 16 + n];
    const int tp = q0 + 4 * g + (n >> 2);
    const uint32_t kt0 = lst[tp], kt1 = lst[tp + 16];
    const lds_cptr kbase = to_lds(bufr<B>().k), vbase = to_lds(bufr<B>().v);
    const lds_cptr ka0 = kbase + (16 * g + kk0 * C::RS), ka1 = kbase + (16 * g + kk1 * C::RS);
    const lds_cptr va0 = vbase + (16 * g + kk0 * C::RS), va1 = vbase + (16 * g + kk1 * C::RS);
    auto ld16 = [](lds_cptr a) { return lds_read16(a); };
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, d0 = s0, d1 = s0;
    if (single) {
#pragma unroll
      for (int sl = 0; sl < C::NSLAB; ++sl) {
        s0 = Mma<bf16_t>::mac8(ld16(ka0 + 64 * sl), qf[sl], s0);
        d0 = Mma<bf16_t>::mac8(ld16(va0 + 64 * sl), df[sl], d0);
      }
    } else {
#pragma unroll
      for (int sl = 0; sl < C::NSLAB; ++sl) {
        const u32x4 a0 = ld16(ka0 + 64 * sl);
        const u32x4 a1 = ld16(ka1 + 64 * sl);
        const u32x4 b0 = ld16(va0 + 64 * sl);
        const u32x4 b1 = ld16(va1 + 64 * sl);
        s0 = Mma<bf16_t>::mac8(a0, qf[sl], s0);
        s1 = Mma<bf16_t>::mac8(a1, qf[sl], s1);
        d0 = Mma<bf16_t>::mac8(b0, df[sl], d0);
        d1 = Mma<bf16_t>::mac8(b1, df[sl], d1);
      }
    }
    bf16x8 sb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float p0 = exp2_fast(__builtin_fmaf(s0[i], cs, -l2));
      float p1 = exp2_fast(__builtin_fmaf(s1[i], cs, -l2));
      if (4 * g + i >= rem) p0 = 0.f;           // padding positions
      if (single || 16 + 4 * g + i >= rem) p1 = 0.f;
      sb[i] = (__bf16)(p0 * (d0[i] - dd));
      sb[4 + i] = (__bf16)(p1 * (d1[i] - dd));
    }
    const u32x4 sbo = __builtin_bit_cast(u32x4, sb);
    // K^T operand: lane (g, n) points at d = 16j + 4(n%4) of the key at
    // position 4g + n/4 of each block and receives d = 16j + n of the four keys
    const lds_cptr ta0 = kbase + (8 * (n & 3) + kt0 * C::RS);
    const lds_cptr ta1 = kbase + (8 * (n & 3) + kt1 * C::RS);
    auto tr = [&](int j) {
      const u32x2 x = lds_read_tr16(ta0 + 32 * j), y = lds_read_tr16(ta1 + 32 * j);
      return u32x4{x[0], x[1], y[0], y[1]};
    };
#pragma unroll
    for (int j = 0; j < C::NDB; ++j) dq[j] = Mma<bf16_t>::mac8(tr(j), sbo, dq[j]);
  }

  // Chunk c from buffer B while chunk c+1 loads into the other buffer.
  template <int B>
  __device__ __forceinline__ void chunk_step(int c, int n_chunks, bool act, int& count) {
    const bool more = c + 1 < n_chunks;
    uint32_t mwn[MW];
    // buffer B^1 was last read in the previous step, which every wave has
    // left.  A wave issues its share of chunk c+1's loads after its first
    // pass (as the dK/dV kernel does), so the compute unit's load queue
    // drains behind matrix-core work instead of stalling every wave at the
    // chunk start.
    bool issued = !more;
    if (act)
      for (int q0 = 0; q0 < count; q0 += 32) {
        pass<B>(q0, count - q0);
        if (!issued) {
          issue_chunk<B ^ 1>(c + 1, mwn);
          issued = true;
        }
      }
    if (!issued) issue_chunk<B ^ 1>(c + 1, mwn);
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
    const size_t head = (size_t)bh * (size_t)L * D;
    kg = reinterpret_cast<const bf16_t*>(p.k) + head;
    vg = reinterpret_cast<const bf16_t*>(p.v) + head;
    const int row0 = qb * C::ROWS + 16 * wave;
    const bool act = row0 < L;
    mrow = p.mask + ((size_t)bh * p.T_q + (size_t)(act ? row0 / p.M : 0)) * p.words;
    const int r = row0 + n;
    const bool rvalid = r < L;
    const int rq = rvalid ? r : L - 1;
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(p.q) + head + (size_t)rq * D;
    const bf16_t* dp = reinterpret_cast<const bf16_t*>(p.dout) + head + (size_t)rq * D;
#pragma unroll
    for (int s = 0; s < C::NSLAB; ++s) {
      qf[s] = *reinterpret_cast<const u32x4*>(qp + 32 * s + 8 * g);
      df[s] = *reinterpret_cast<const u32x4*>(dp + 32 * s + 8 * g);
    }
    if (!rvalid)
#pragma unroll
      for (int s = 0; s < C::NSLAB; ++s) {
        qf[s] = u32x4{0u, 0u, 0u, 0u};
        df[s] = u32x4{0u, 0u, 0u, 0u};
      }
    cs = p.cs;
    if (p.scale < 0.f)
#pragma unroll
      for (int s = 0; s < C::NSLAB; ++s) qf[s] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    const float* ldr = p.ld + ((size_t)bh * p.n_qc + (size_t)(rq / kBwdChunk)) * 256 + (rq % kBwdChunk);
    l2 = rvalid ? ldr[0] : INFINITY;
    dd = rvalid ? ldr[kBwdChunk] : 0.f;
#pragma unroll
    for (int s = 0; s < C::NSLAB; ++s) {
      asm volatile("" : "+v"(qf[s]));
      asm volatile("" : "+v"(df[s]));
    }
    asm volatile("" : "+v"(l2), "+v"(dd));
#pragma unroll
    for (int j = 0; j < C::NDB; ++j) dq[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int n_chunks = (L + C::KC - 1) / C::KC;
#pragma unroll
    for (int u = 0; u < NK_W; ++u) {
      const int j = wave + C::W * u;
      koff[u] = dma_offset(j < C::NI_T ? j : 0, lane, C::KC);
    }
    uint32_t mw[MW];
    issue_chunk<0>(0, mw);
    __builtin_amdgcn_s_waitcnt(0);
    int count = act ? make_list(0, mw) : 0;
    __syncthreads();
    // two chunks per iteration, so that each step names its buffer statically
    for (int c = 0; c < n_chunks; c += 2) {
      chunk_step<0>(c, n_chunks, act, count);
      if (c + 1 < n_chunks) chunk_step<1>(c + 1, n_chunks, act, count);
    }

    if (!rvalid) return;
    bf16_t* dqg = reinterpret_cast<bf16_t*>(p.dq) + head + (size_t)r * D;
#pragma unroll
    for (int j = 0; j < C::NDB; ++j) {
      bf16x4 a;
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = (__bf16)(dq[j][i] * p.scale);
      *reinterpret_cast<u32x2*>(dqg + 16 * j + 4 * g) = __builtin_bit_cast(u32x2, a);
    }
  }
};

template <int D, int N>
__global__ __launch_bounds__((64 * DqCfg<D, N>::W)) void bwd_dq_kernel(BwdParams p) {
  using K = DqKernel<D, N>;
  __shared__ __attribute__((aligned(16))) typename K::Buf b0;
  __shared__ __attribute__((aligned(16))) typename K::Buf b1;
  __shared__ __attribute__((aligned(16))) typename K::Lists lists;
  K k(p, b0, b1, lists);
  k.run();
}

}  // namespace tsa
