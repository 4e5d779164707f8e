// Global-to-LDS staging rates on gfx950: direct loads into LDS
// (buffer_load ... lds, 1 KB per wave instruction) against loads into
// registers followed by LDS stores, with the source resident in L2.  Each
// wave moves `kLoads` 1-KB blocks per round and waits for them at the end of
// the round, like one chunk of the attention kernel's staging.  All
// addresses are in bounds and every kernel runs a fixed number of rounds.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops micro/dma_rates.hip -o dma_rates
//   ./dma_rates
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

constexpr int kRounds = 512;
constexpr int kSrcBytes = 1 << 20;   // 1 MB source, L2-resident after the first round
constexpr int kWaves = 16;

// LOADS direct 1-KB loads per wave per round into a 64-KB LDS area.
template <int LOADS>
__global__ __launch_bounds__(64 * kWaves) void dma_lds(const unsigned char* __restrict__ src, unsigned* out) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[65536];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, kSrcBytes, 0x00020000);
  for (int r = 0; r < kRounds; ++r) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int blk = (wave * LOADS + u) & 63;                       // 64 KB of LDS
      const unsigned off = (unsigned)(((blockIdx.x * 97 + r * 61 + wave * LOADS + u) & 1023) * 1024 + 16 * lane);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(lds + blk * 1024), 16, off, 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (lane == 64) out[0] = lds[threadIdx.x];
}

// The same traffic through registers: global loads, wait, LDS stores.
template <int LOADS>
__global__ __launch_bounds__(64 * kWaves) void via_vgpr(const unsigned char* __restrict__ src, unsigned* out) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[65536];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int r = 0; r < kRounds; ++r) {
    u32x4 x[LOADS];
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const unsigned off = (unsigned)(((blockIdx.x * 97 + r * 61 + wave * LOADS + u) & 1023) * 1024 + 16 * lane);
      x[u] = *reinterpret_cast<const u32x4*>(src + off);
    }
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int blk = (wave * LOADS + u) & 63;
      *reinterpret_cast<u32x4*>(lds + blk * 1024 + 16 * lane) = x[u];
    }
    __syncthreads();
  }
  if (lane == 64) out[0] = lds[threadIdx.x];
}

template <typename F>
float time_ms(F launch) {
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  launch();
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(a));
  for (int r = 0; r < 3; ++r) launch();
  CHECK(hipEventRecord(b));
  CHECK(hipEventSynchronize(b));
  float ms;
  CHECK(hipEventElapsedTime(&ms, a, b));
  return ms / 3;
}

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  const double clk = 2.4e9;
  unsigned char* src;
  unsigned* out;
  CHECK(hipMalloc(&src, kSrcBytes));
  CHECK(hipMemset(src, 1, kSrcBytes));
  CHECK(hipMalloc(&out, 64));
  const int blocks = cus;  // one 1024-thread work-group per CU (64 KB of LDS each)
  auto rate = [&](int loads, float ms) {
    const double bytes = (double)blocks * kWaves * loads * 1024.0 * kRounds;
    return bytes / (ms * 1e-3) / clk / cus;
  };
  float t;
  t = time_ms([&] { hipLaunchKernelGGL(dma_lds<4>, dim3(blocks), dim3(64 * kWaves), 0, 0, src, out); });
  printf("LDS-direct loads, 4 KB per wave per round  : %6.1f B/clk/CU (%.3f ms)\n", rate(4, t), t);
  t = time_ms([&] { hipLaunchKernelGGL(dma_lds<8>, dim3(blocks), dim3(64 * kWaves), 0, 0, src, out); });
  printf("LDS-direct loads, 8 KB per wave per round  : %6.1f B/clk/CU (%.3f ms)\n", rate(8, t), t);
  t = time_ms([&] { hipLaunchKernelGGL(via_vgpr<4>, dim3(blocks), dim3(64 * kWaves), 0, 0, src, out); });
  printf("registers + LDS stores, 4 KB per wave/round: %6.1f B/clk/CU (%.3f ms)\n", rate(4, t), t);
  t = time_ms([&] { hipLaunchKernelGGL(via_vgpr<8>, dim3(blocks), dim3(64 * kWaves), 0, 0, src, out); });
  printf("registers + LDS stores, 8 KB per wave/round: %6.1f B/clk/CU (%.3f ms)\n", rate(8, t), t);
  CHECK(hipFree(src));
  CHECK(hipFree(out));
  return 0;
}
