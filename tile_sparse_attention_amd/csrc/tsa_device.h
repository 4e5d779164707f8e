// Device-side helpers shared by the tile-sparse attention kernels (gfx950).
//
// Wave64 throughout.  Matrix-core operand layouts used here (CDNA3/CDNA4
// MFMA, 16x16 output block): for lane l, let g = l / 16 and n = l % 16;
//   A (16 x K): lane holds row n, k-elements of group g;
//   B (K x 16): lane holds column n, k-elements of group g;
//   D (16 x 16, fp32): lane holds D[4g + i][n], i = 0..3.
// Which k-values a group holds only has to agree between A and B, so every
// kernel picks the k order that makes its loads contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

typedef uint16_t bf16_t;  // storage type of bf16 elements in memory

// Fourth word of a raw (unformatted, unswizzled) buffer resource on gfx9.
constexpr int kBufferFlags = 0x00020000;

// One-dimensional launches over many items: a dispatch holds fewer than 2^32
// work-items in each grid dimension, so such kernels take at most
// kMaxStrideBlocks work-groups and step through their items with a stride
// of gridDim.x work-groups.
constexpr long long kMaxStrideBlocks = 1ll << 20;
inline unsigned stride_blocks(long long items, long long per_block) {
  const long long b = (items + per_block - 1) / per_block;
  return (unsigned)(b < 1 ? 1 : b < kMaxStrideBlocks ? b : kMaxStrideBlocks);
}

__device__ __forceinline__ int lane_id() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Number of set bits of `m` strictly below this lane (wave64 prefix count).
__device__ __forceinline__ uint32_t prefix_count64(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Lane 0's value of a 32-bit word, zero-extended (readfirstlane is int-typed).
__device__ __forceinline__ uint32_t uniform_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}

// Wave-level compaction of one 64-tile window of a keep-bitmap row.
// `bits` is wave-uniform: bit t keeps tile (base + t).  Every lane t whose bit
// is set stores (base + t) at position `offset + (set bits below t)` through
// `store(pos, value)`.  Returns the number of set bits.  The result list is
// ascending because positions follow bit order.
template <typename Store>
__device__ __forceinline__ uint32_t wave_compact64(uint64_t bits, int base, uint32_t offset,
                                                   Store&& store) {
  const int t = lane_id();
  if ((bits >> t) & 1ull) store(offset + prefix_count64(bits), base + t);
  return (uint32_t)__builtin_popcountll(bits);
}

// Bits [first, first + count) of a bitmap row as a 64-bit value (count <= 64,
// `first` a multiple of `count`, count a power of two).  Bits at or beyond
// `valid` (the row's real tile count) are cleared.
// Only words holding at least one valid bit are read.
__device__ __forceinline__ uint64_t row_bits(const uint32_t* __restrict__ row, int first, int count,
                                             int valid) {
  const int room = valid - first;
  if (room <= 0) return 0ull;
  uint64_t b;
  if (count <= 32) {
    const uint32_t w = row[first >> 5];
    const uint64_t lo = (uint64_t)(w >> (first & 31));
    b = count == 32 ? lo : (lo & ((1ull << count) - 1ull));
  } else {
    b = (uint64_t)row[first >> 5];
    if (room > 32) b |= (uint64_t)row[(first >> 5) + 1] << 32;
  }
  if (room < count) b &= (1ull << room) - 1ull;
  return b;
}

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}

// Exchange with the lane whose index differs in bit 4 / bit 5 (ds_bpermute).
__device__ __forceinline__ float xor_lane16(float x) { return __shfl_xor(x, 16); }
__device__ __forceinline__ float xor_lane32(float x) { return __shfl_xor(x, 32); }

// Work-groups of a 1-D grid are handed to the eight XCDs of the chip in
// turn (block b to XCD b mod 8), and each XCD has an L2 of its own.  This
// renumbering gives every XCD one contiguous range of logical blocks, in
// dispatch order: blocks that run together on an XCD are consecutive logical
// blocks (of the same head, for the attention grid) and share its L2.
__device__ __forceinline__ int xcd_major_block(int b, int nb) {
  constexpr int X = 8;
  const int x = b % X, i = b / X;
  const int q = nb / X, r = nb % X;
  return x * q + (x < r ? x : r) + i;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS byte address of a pointer into a __shared__ array, and a typed LDS
// load from such an address (integer address arithmetic keeps the per-pass
// index math to one multiply-add or shift-add per address).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
template <typename T>
__device__ __forceinline__ T lds_load(uint32_t a) {
  return *(const __attribute__((address_space(3))) T*)(uintptr_t)a;
}

// LDS reads through 32-bit pointers that keep the __shared__ object they
// point into.  Direct global-to-LDS loads in flight write LDS behind the
// compiler's back, so before an LDS read it waits for every such load it
// cannot prove writes elsewhere; with double buffers as two separate objects
// and reads through pointers into them, a read of one buffer does not wait
// for the loads into the other.
typedef const __attribute__((address_space(3))) uint8_t* lds_cptr;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ __forceinline__ lds_cptr to_lds(const uint8_t* p) { return (lds_cptr)p; }
__device__ __forceinline__ u32x4 lds_read16(lds_cptr a) {
  return *(const __attribute__((address_space(3))) u32x4*)a;
}
__device__ __forceinline__ u32x2 lds_read8(lds_cptr a) {
  return *(const __attribute__((address_space(3))) u32x2*)a;
}
// Transposing read (16-bit elements): within each 16-lane group, lane s
// points at 4 consecutive elements of row s>>2 of a 4-row block; lane n of
// the group receives element n of each of the four rows (column n of the
// 16-column block the four lanes of a row cover).
__device__ __forceinline__ u32x2 lds_read_tr16(lds_cptr a) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a));
}

// Direct global-to-LDS loads of a staged tile cut into NP pieces of 1 KB (16
// bytes per lane): a wave issues pieces wave, wave + W, ... below NP, each from
// buffer resource r at its lanes' source offsets off[u] (computed once by the
// caller) into piece j of the LDS tile at dst.  Every wave takes the same
// static slots, so no load picks its tile or computes its offset at run time.
template <int NP, int W>
__device__ __forceinline__ void load_pieces(__amdgpu_buffer_rsrc_t r, __attribute__((address_space(3))) uint8_t* dst,
                                            const uint32_t (&off)[(NP + W - 1) / W], int wave) {
  constexpr int NS = (NP + W - 1) / W;
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int j = wave + W * u;
    if (NP % W == 0 || u + 1 < NS || j < NP) {
      const uint32_t o = off[u];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + j * 1024), 16, o,
                                               0, 0, 0);
    }
  }
}

// a * b + c (24-bit operands, b wave-uniform) and (a << 4) + c as single
// instructions; the compiler otherwise splits both into two.
__device__ __forceinline__ uint32_t mad_u24(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(b), "v"(c));
  return r;
}
__device__ __forceinline__ uint32_t shl4_add(uint32_t a, uint32_t c) {
  uint32_t r;
  asm("v_lshl_add_u32 %0, %1, 4, %2" : "=v"(r) : "v"(a), "v"(c));
  return r;
}

// Maximum over lanes l, l^16, l^32 and l^48 (the four 16-lane rows of the
// wave), with two lane swaps and no LDS traffic.
__device__ __forceinline__ float max_across_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// A zero the compiler cannot see through: adding it to an index keeps a
// loop-invariant computation inside the loop (recomputed, not kept live).
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  return z;
}

}  // namespace tsa
