// Does vector ALU work overlap bf16 MFMA work on one gfx950 SIMD?  Each wave
// runs a loop of independent 16x16x32 bf16 MFMAs interleaved with a fixed
// number of independent fp32 FMAs (or v_exp_f32) per MFMA, optionally with a
// 16-byte-per-lane LDS read per MFMA (the attention passes' operand feed).
// The time per loop against the MFMA-only and VALU-only times tells whether
// the matrix core and the VALU run concurrently.  All LDS addresses are in
// bounds and every loop has a fixed trip count.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops micro/mix.hip -o mix
//   ./mix
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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kIters = 2048;  // MFMAs per wave

// MFMA = MFMAs per loop step (0 or 4), VALU = fp32 FMAs per step, EXP =
// v_exp_f32 per step, LDS = 16-byte LDS reads per step (each feeds one MFMA
// when MFMA > 0).
template <int THREADS, int MFMA, int VALU, int EXP, int LDS>
__global__ __launch_bounds__(THREADS) void mix(unsigned* out, float seed) {
  __shared__ __attribute__((aligned(16))) unsigned lds[8192];  // 32 KB
  if (LDS > 0) {
    for (int i = threadIdx.x; i < 8192; i += THREADS) lds[i] = 0x3f803f80u + (i & 7);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int wv = (threadIdx.x >> 6) & 7;
  // rows 288 bytes apart, lane groups 16 bytes apart: a conflict-free pattern
  const char* lb = reinterpret_cast<const char*>(lds) + (lane & 15) * 288 + (lane >> 4) * 16 + wv * 64;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(seed * i); b[i] = (__bf16)(seed + i); }
  f32x4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = seed * (threadIdx.x + i);
  for (int it = 0; it < kIters / 4; ++it) {
    bf16x8 op[4] = {a, a, a, a};
    if (LDS > 0) {
      asm volatile("" ::: "memory");
      const char* p = lb + ((it * 4096) & 16383);
#pragma unroll
      for (int u = 0; u < LDS; ++u) op[u & 3] = *reinterpret_cast<const bf16x8*>(p + u * 4608);
    }
    if (MFMA > 0) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[0], b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[1], b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[2], b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[3], b, c3, 0, 0, 0);
    } else if (LDS > 0) {
      c0[0] += (float)op[0][0]; c1[0] += (float)op[1][1]; c2[0] += (float)op[2][2]; c3[0] += (float)op[3][3];
    }
#pragma unroll
    for (int v = 0; v < 4 * VALU; ++v) x[v & 7] = __builtin_fmaf(x[v & 7], 0.999f, 0.5f);
#pragma unroll
    for (int v = 0; v < 4 * EXP; ++v) x[v & 7] = __builtin_amdgcn_exp2f(x[v & 7]);
  }
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += x[i];
  const f32x4 t = c0 + c1 + c2 + c3;
  if (s + t.x + t.y + t.z + t.w == 1.2345f) out[0] = 1;
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

unsigned* g_out;
int g_cus;

// cycles per MFMA slot per SIMD: total SIMD-cycles / (waves per SIMD * MFMAs per wave)
template <int THREADS, int MFMA, int VALU, int EXP, int LDS>
void run(const char* what) {
  const int blocks = g_cus * (1024 / THREADS);  // 16 waves per CU = 4 per SIMD
  float t = time_ms([&] {
    hipLaunchKernelGGL((mix<THREADS, MFMA, VALU, EXP, LDS>), dim3(blocks), dim3(THREADS), 0, 0, g_out, 0.01f);
  });
  const double clk = 2.4e9;
  const double simd_cycles = t * 1e-3 * clk;            // every SIMD runs the whole time
  const double per_step = simd_cycles / (4.0 * kIters); // 4 waves per SIMD, kIters MFMA slots per wave
  printf("%-44s: %6.2f SIMD cycles per MFMA slot (%.3f ms)\n", what, per_step, t);
}

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  g_cus = prop.multiProcessorCount;
  CHECK(hipMalloc(&g_out, 64));
  printf("device %s, %d CUs, 4 waves per SIMD, %d MFMA slots per wave\n", prop.name, g_cus, kIters);
  run<1024, 1, 0, 0, 0>("MFMA only");
  run<1024, 0, 1, 0, 0>("1 FMA only");
  run<1024, 0, 4, 0, 0>("4 FMA only");
  run<1024, 0, 0, 1, 0>("1 exp only");
  run<1024, 1, 1, 0, 0>("MFMA + 1 FMA");
  run<1024, 1, 2, 0, 0>("MFMA + 2 FMA");
  run<1024, 1, 3, 0, 0>("MFMA + 3 FMA");
  run<1024, 1, 4, 0, 0>("MFMA + 4 FMA");
  run<1024, 1, 0, 1, 0>("MFMA + 1 exp");
  run<1024, 1, 2, 1, 0>("MFMA + 2 FMA + 1 exp");
  run<1024, 0, 0, 0, 4>("1 KB LDS only");
  run<1024, 1, 0, 0, 4>("MFMA + 1 KB LDS");
  run<1024, 1, 2, 0, 4>("MFMA + 1 KB LDS + 2 FMA");
  run<1024, 1, 2, 1, 4>("MFMA + 1 KB LDS + 2 FMA + 1 exp");
  CHECK(hipFree(g_out));
  return 0;
}
