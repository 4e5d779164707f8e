// Per-CU throughput microbenchmarks for the resources the tile-sparse
// attention kernel depends on (gfx950): LDS reads (b128, b64, transposing
// b64), bf16 16x16x32 / 16x16x16 and FP8 16x16x32 / 16x16x128 MFMA,
// v_exp_f32 and fp32 FMA.  Every kernel is
// in-bounds and exits after a fixed number of iterations.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops micro/rates.hip -o micro_rates
//   ./micro_rates
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));              \
      exit(1);                                                                    \
    }                                                                             \
  } while (0)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kIters = 4096;

// Each lane reads 16 bytes at lane*16 + ((it*1024) mod 32 KB): consecutive
// lanes, consecutive 16-byte slots (conflict-free).
__global__ __launch_bounds__(kThreads) void lds_b128(unsigned* out) {
  __shared__ __attribute__((aligned(16))) unsigned lds[16384];  // 64 KB
  for (int i = threadIdx.x; i < 16384; i += kThreads) lds[i] = i;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  u32x4 acc = {0, 0, 0, 0};
  for (int it = 0; it < kIters; ++it) {
    const int off = (lane * 16 + ((it * 1024 + (threadIdx.x >> 6) * 4096) & 32767)) >> 2;
    acc ^= *reinterpret_cast<const u32x4*>(&lds[off]);
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x12345678u) out[0] = 1;
}

__global__ __launch_bounds__(kThreads) void lds_b64(unsigned* out) {
  __shared__ __attribute__((aligned(16))) unsigned lds[16384];
  for (int i = threadIdx.x; i < 16384; i += kThreads) lds[i] = i;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  u32x2 acc = {0, 0};
  for (int it = 0; it < kIters; ++it) {
    const int off = (lane * 8 + ((it * 512 + (threadIdx.x >> 6) * 4096) & 32767)) >> 2;
    acc ^= *reinterpret_cast<const u32x2*>(&lds[off]);
  }
  if ((acc.x ^ acc.y) == 0x12345678u) out[0] = 1;
}

// Transposing read: lanes 4j..4j+3 of each 16-lane block read row j (4 rows of
// 32 bytes per block, rows 272 bytes apart), as an MFMA operand gather would.
__global__ __launch_bounds__(kThreads) void lds_tr16(unsigned* out) {
  __shared__ __attribute__((aligned(16))) unsigned short lds[32768];
  for (int i = threadIdx.x; i < 32768; i += kThreads) lds[i] = (unsigned short)i;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int blk = lane >> 4, j = (lane >> 2) & 3, c = lane & 3;
  i16x4 acc = {0, 0, 0, 0};
  for (int it = 0; it < kIters; ++it) {
    const int row = (blk * 4 + j + (it & 15) * 16 + (threadIdx.x >> 6) * 4) & 127;
    const int off = row * 136 + c * 4 + ((it >> 4) & 7) * 16;
    acc ^= __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(lds + off));
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x1234) out[0] = 1;
}


// Eight independent reads in flight per wave, each result consumed by an
// empty asm statement (no VALU work in the loop).  32 KB of LDS per
// work-group, four work-groups (16 waves) per CU.  PAT 0: consecutive lanes
// read consecutive 16-byte slots; PAT 1: the MFMA-operand pattern of the
// attention kernel (lane (g, n) reads 16 bytes at byte 16*g of row n, rows
// 272 bytes apart).
template <int PAT>
__global__ __launch_bounds__(kThreads) void lds_b128_ilp(unsigned* out) {
  __shared__ __attribute__((aligned(16))) unsigned lds[8192];  // 32 KB
  for (int i = threadIdx.x; i < 8192; i += kThreads) lds[i] = i;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int base = (PAT == 0 ? lane * 16 : (lane & 15) * 272 + (lane >> 4) * 16) + wv * 1024;
  const char* lb = reinterpret_cast<const char*>(lds) + base;
  for (int it = 0; it < kIters / 8; ++it) {
    const char* p = lb + ((it * 2048) & 8191);
    u32x4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const u32x4*>(p + u * 1024);
    asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]),
                 "v"(x[7]));
  }
  if (lane == 64) out[0] = 1;
}

// LDS operand feed of the attention passes: every 16x16x32 MFMA takes one
// operand from a 16-byte-per-lane LDS read (1 KB per MFMA), the other from
// registers.  Reports the MFMA rate reached.
__global__ __launch_bounds__(kThreads) void mix_lds_mfma(unsigned* out, float seed) {
  __shared__ __attribute__((aligned(16))) unsigned lds[8192];  // 32 KB
  for (int i = threadIdx.x; i < 8192; i += kThreads) lds[i] = 0x3f803f80u + (i & 7);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const char* lb = reinterpret_cast<const char*>(lds) + (lane & 15) * 272 + (lane >> 4) * 16 + wv * 1024;
  bf16x8 b;
  for (int i = 0; i < 8; ++i) b[i] = (__bf16)(seed + i);
  f32x4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
  for (int it = 0; it < kIters / 8; ++it) {
    asm volatile("" ::: "memory");  // keeps the reads in the loop
    const char* p = lb + ((it * 2048) & 8191);
#pragma unroll
    for (int u = 0; u < 8; u += 4) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(p + u * 1024);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(p + u * 1024 + 1024);
      const bf16x8 a2 = *reinterpret_cast<const bf16x8*>(p + u * 1024 + 2048);
      const bf16x8 a3 = *reinterpret_cast<const bf16x8*>(p + u * 1024 + 3072);
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a3, b, c3, 0, 0, 0);
    }
  }
  const f32x4 s = c0 + c1 + c2 + c3;
  if (s.x + s.y + s.z + s.w == 1.2345f) out[0] = 1;
}

// Vector-memory reads of an L1/L2-resident 16 KB block per work-group
// (global_load_dwordx4, 8 independent loads in flight per wave).
__global__ __launch_bounds__(kThreads) void l1_b128_ilp(const unsigned* __restrict__ src, unsigned* out) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const unsigned* blk = src + (blockIdx.x & 63) * 4096;  // 64 distinct 16 KB blocks
  u32x4 acc[8];
  for (int u = 0; u < 8; ++u) acc[u] = u32x4{0, 0, 0, 0};
  for (int it = 0; it < kIters / 8; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int off = (lane * 16 + (((it * 8 + u) * 1024 + wv * 4096) & 16383)) >> 2;
      acc[u] ^= *reinterpret_cast<const u32x4*>(&blk[off]);
    }
  }
  u32x4 a = acc[0];
  for (int u = 1; u < 8; ++u) a ^= acc[u];
  if ((a.x ^ a.y ^ a.z ^ a.w) == 0x12345678u) out[0] = 1;
}


// LDS read pattern probe: lane (g, n) = (lane >> gshift, lane & (2^gshift - 1))
// reads W bytes at n*rstride + g*gstride (+ 256-byte multiples that keep the
// bank mapping), eight reads in flight.  Profiled with the LDS bank-conflict
// counter, it shows which operand layouts the LDS serves conflict-free.
template <int W>
__global__ __launch_bounds__(kThreads) void lds_pattern(unsigned* out, int rstride, int gstride,
                                                        int gshift) {
  __shared__ __attribute__((aligned(16))) unsigned lds[8192];  // 32 KB
  for (int i = threadIdx.x; i < 8192; i += kThreads) lds[i] = i;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int n = lane & ((1 << gshift) - 1), g = lane >> gshift;
  const char* lb = reinterpret_cast<const char*>(lds) + n * rstride + g * gstride + wv * 4096;
  for (int it = 0; it < kIters / 8; ++it) {
    asm volatile("" ::: "memory");
    if constexpr (W == 16) {
      u32x4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const u32x4*>(lb + u * 256);
      asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]),
                   "v"(x[7]));
    } else {
      u32x2 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const u32x2*>(lb + u * 256);
      asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]),
                   "v"(x[7]));
    }
  }
  if (lane == 64) out[0] = 1;
}

__global__ __launch_bounds__(kThreads) void mfma_bf16(unsigned* out, float seed) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(seed * i); b[i] = (__bf16)(seed + i); }
  f32x4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
  for (int it = 0; it < kIters / 4; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
  }
  const f32x4 s = c0 + c1 + c2 + c3;
  if (s.x + s.y + s.z + s.w == 1.2345f) out[0] = 1;
}


__global__ __launch_bounds__(kThreads) void mfma_bf16_k16(unsigned* out, float seed) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 a, b;
  for (int i = 0; i < 4; ++i) { a[i] = (__bf16)(seed * i); b[i] = (__bf16)(seed + i); }
  f32x4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
  for (int it = 0; it < kIters / 4; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c3, 0, 0, 0);
  }
  const f32x4 s = c0 + c1 + c2 + c3;
  if (s.x + s.y + s.z + s.w == 1.2345f) out[0] = 1;
}

// FP8 (e4m3) steps: the 32-deep one that gfx950 inherits and its 128-deep
// one (block scales 2^0)
__global__ __launch_bounds__(kThreads) void mfma_fp8_k32(unsigned* out, float seed) {
  const long a = (long)(seed * 1000.f) * 0x0101010101010101L, b = a ^ 0x1122334455667788L;
  f32x4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
  for (int it = 0; it < kIters / 4; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c3, 0, 0, 0);
  }
  const f32x4 s = c0 + c1 + c2 + c3;
  if (s.x + s.y + s.z + s.w == 1.2345f) out[0] = 1;
}

__global__ __launch_bounds__(kThreads) void mfma_fp8_k128(unsigned* out, float seed) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  i32x8 a, b;
  for (int i = 0; i < 8; ++i) { a[i] = (int)(seed * 1000.f) * (i + 1); b[i] = a[i] ^ 0x11223344; }
  f32x4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
  for (int it = 0; it < kIters / 4; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c1, 0, 0, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c2, 0, 0, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c3, 0, 0, 0, 127, 0, 127);
  }
  const f32x4 s = c0 + c1 + c2 + c3;
  if (s.x + s.y + s.z + s.w == 1.2345f) out[0] = 1;
}

__global__ __launch_bounds__(kThreads) void valu_exp(unsigned* out, float seed) {
  float x0 = seed * threadIdx.x, x1 = x0 + 1.f, x2 = x0 + 2.f, x3 = x0 + 3.f;
  for (int it = 0; it < kIters / 4; ++it) {
    x0 = __builtin_amdgcn_exp2f(x0); x1 = __builtin_amdgcn_exp2f(x1);
    x2 = __builtin_amdgcn_exp2f(x2); x3 = __builtin_amdgcn_exp2f(x3);
  }
  if (x0 + x1 + x2 + x3 == 1.2345f) out[0] = 1;
}

__global__ __launch_bounds__(kThreads) void valu_fma(unsigned* out, float seed) {
  float x0 = seed * threadIdx.x, x1 = x0 + 1.f, x2 = x0 + 2.f, x3 = x0 + 3.f;
  for (int it = 0; it < kIters / 4; ++it) {
    x0 = __builtin_fmaf(x0, 0.999f, 0.5f); x1 = __builtin_fmaf(x1, 0.999f, 0.5f);
    x2 = __builtin_fmaf(x2, 0.999f, 0.5f); x3 = __builtin_fmaf(x3, 0.999f, 0.5f);
  }
  if (x0 + x1 + x2 + x3 == 1.2345f) out[0] = 1;
}

template <typename F>
float time_ms(F launch) {
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  launch();
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(a));
  for (int r = 0; r < 5; ++r) launch();
  CHECK(hipEventRecord(b));
  CHECK(hipEventSynchronize(b));
  float ms;
  CHECK(hipEventElapsedTime(&ms, a, b));
  return ms / 5;
}

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  const double clk = 2.4e9;  // peak engine clock of MI355X
  unsigned* out;
  CHECK(hipMalloc(&out, 64));
  const int blocks = cus * 8;
  const double waves = (double)blocks * kThreads / 64;
  printf("device %s, %d CUs, %d blocks x %d threads, %d iterations\n", prop.name, cus, blocks,
         kThreads, kIters);
  auto per_cu_clk = [&](double total, float ms) { return total / (ms * 1e-3) / clk / cus; };
  float t;
  t = time_ms([&] { hipLaunchKernelGGL(lds_b128, dim3(blocks), dim3(kThreads), 0, 0, out); });
  printf("ds_read_b128      : %7.1f B/clk/CU (%.3f ms)\n", per_cu_clk(waves * 64 * 16 * kIters, t), t);
  t = time_ms([&] { hipLaunchKernelGGL(lds_b64, dim3(blocks), dim3(kThreads), 0, 0, out); });
  printf("ds_read_b64       : %7.1f B/clk/CU (%.3f ms)\n", per_cu_clk(waves * 64 * 8 * kIters, t), t);
  t = time_ms([&] { hipLaunchKernelGGL(lds_tr16, dim3(blocks), dim3(kThreads), 0, 0, out); });
  printf("ds_read_b64_tr_b16: %7.1f B/clk/CU (%.3f ms)\n", per_cu_clk(waves * 64 * 8 * kIters, t), t);
  t = time_ms([&] { hipLaunchKernelGGL(lds_b128_ilp<0>, dim3(blocks), dim3(kThreads), 0, 0, out); });
  printf("ds_read_b128 x8   : %7.1f B/clk/CU (%.3f ms) consecutive slots\n",
         per_cu_clk(waves * 64 * 16 * (kIters / 8) * 8, t), t);
  t = time_ms([&] { hipLaunchKernelGGL(lds_b128_ilp<1>, dim3(blocks), dim3(kThreads), 0, 0, out); });
  printf("ds_read_b128 x8   : %7.1f B/clk/CU (%.3f ms) MFMA operand rows, 272-byte stride\n",
         per_cu_clk(waves * 64 * 16 * (kIters / 8) * 8, t), t);
  t = time_ms([&] { hipLaunchKernelGGL(mix_lds_mfma, dim3(blocks), dim3(kThreads), 0, 0, out, 0.5f); });
  printf("mfma + 1 KB LDS   : %7.1f FLOP/clk/CU (%.3f ms), %.1f B/clk/CU of LDS reads\n",
         per_cu_clk(waves * (kIters / 8) * 8 * 16.0 * 16 * 32 * 2, t), t,
         per_cu_clk(waves * (kIters / 8) * 8 * 1024.0, t));
  unsigned* src;
  CHECK(hipMalloc(&src, 64 * 16384));
  CHECK(hipMemset(src, 1, 64 * 16384));
  t = time_ms([&] { hipLaunchKernelGGL(l1_b128_ilp, dim3(blocks), dim3(kThreads), 0, 0, src, out); });
  printf("global b128 x8    : %7.1f B/clk/CU (%.3f ms) cache-resident 16 KB blocks\n",
         per_cu_clk(waves * 64 * 16 * (kIters / 8) * 8, t), t);
  CHECK(hipFree(src));
  {
    struct Pat { int w, rs, gs, gsh; const char* what; };
    const Pat pats[] = {
        {16, 16, 0, 6, "b128 consecutive"},
        {16, 272, 16, 4, "b128 rows 272 B apart, groups 16 B"},
        {16, 256, 16, 4, "b128 rows 256 B apart, groups 16 B"},
        {16, 272, 64, 4, "b128 rows 272 B apart, groups 64 B"},
        {16, 288, 16, 4, "b128 rows 288 B apart, groups 16 B"},
        {16, 264, 16, 4, "b128 rows 264 B apart, groups 16 B"},
        {16, 16, 256, 3, "b128 8 rows x 16 B consecutive, groups 256 B"},
        {16, 272, 16, 3, "b128 8 rows 272 B apart, groups 16 B"},
        {8, 8, 0, 6, "b64 consecutive"},
        {8, 272, 8, 4, "b64 rows 272 B apart, groups 8 B"},
        {8, 272, 16, 4, "b64 rows 272 B apart, groups 16 B"},
        {8, 264, 8, 4, "b64 rows 264 B apart, groups 8 B"},
    };
    for (const Pat& q : pats) {
      if (q.w == 16)
        t = time_ms([&] { hipLaunchKernelGGL(lds_pattern<16>, dim3(blocks), dim3(kThreads), 0, 0, out, q.rs, q.gs, q.gsh); });
      else
        t = time_ms([&] { hipLaunchKernelGGL(lds_pattern<8>, dim3(blocks), dim3(kThreads), 0, 0, out, q.rs, q.gs, q.gsh); });
      printf("pattern %-48s: %7.1f B/clk/CU (%.3f ms)\n", q.what,
             per_cu_clk(waves * 64.0 * q.w * (kIters / 8) * 8, t), t);
    }
  }
  t = time_ms([&] { hipLaunchKernelGGL(mfma_bf16, dim3(blocks), dim3(kThreads), 0, 0, out, 0.5f); });
  printf("mfma 16x16x32 bf16: %7.1f FLOP/clk/CU (%.3f ms)\n",
         per_cu_clk(waves * kIters * 16.0 * 16 * 32 * 2, t), t);
  t = time_ms([&] { hipLaunchKernelGGL(mfma_bf16_k16, dim3(blocks), dim3(kThreads), 0, 0, out, 0.5f); });
  printf("mfma 16x16x16 bf16: %7.1f FLOP/clk/CU (%.3f ms)\n",
         per_cu_clk(waves * kIters * 16.0 * 16 * 16 * 2, t), t);
  t = time_ms([&] { hipLaunchKernelGGL(mfma_fp8_k32, dim3(blocks), dim3(kThreads), 0, 0, out, 0.5f); });
  printf("mfma 16x16x32 fp8 : %7.1f FLOP/clk/CU (%.3f ms)\n",
         per_cu_clk(waves * kIters * 16.0 * 16 * 32 * 2, t), t);
  t = time_ms([&] { hipLaunchKernelGGL(mfma_fp8_k128, dim3(blocks), dim3(kThreads), 0, 0, out, 0.5f); });
  printf("mfma 16x16x128 f8 : %7.1f FLOP/clk/CU (%.3f ms)\n",
         per_cu_clk(waves * kIters * 16.0 * 16 * 128 * 2, t), t);
  t = time_ms([&] { hipLaunchKernelGGL(valu_exp, dim3(blocks), dim3(kThreads), 0, 0, out, 0.01f); });
  printf("v_exp_f32         : %7.1f lane-ops/clk/CU (%.3f ms)\n", per_cu_clk(waves * 64 * kIters, t), t);
  t = time_ms([&] { hipLaunchKernelGGL(valu_fma, dim3(blocks), dim3(kThreads), 0, 0, out, 0.01f); });
  printf("v_fma_f32         : %7.1f lane-ops/clk/CU (%.3f ms)\n", per_cu_clk(waves * 64 * kIters, t), t);
  CHECK(hipFree(out));
  return 0;
}
