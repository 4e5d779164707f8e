// How much does staging data into LDS slow concurrent LDS operand reads on
// gfx950?  Sixteen waves per work-group (one work-group per CU) loop over
// conflict-free 16-byte-per-lane LDS reads (eight per step, 8 KB per wave);
// every STAGE-th step each wave also moves 1 KB from an L2-resident buffer
// into LDS, either with a direct global-to-LDS load or through registers
// (global load + LDS store), or only loads it into registers.  All
// addresses are in bounds and every loop has a fixed trip count.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops micro/lds_interference.hip -o lds_interference
//   ./lds_interference
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

constexpr int kSteps = 2048;
constexpr int kSrcBytes = 1 << 20;
constexpr int kWaves = 16;

// MODE 0: reads only; 1: direct global->LDS load; 2: global load + LDS
// store; 3: global load into registers only.
template <int MODE, int STAGE>
__global__ __launch_bounds__(64 * kWaves) void interfere(const unsigned char* __restrict__ src, unsigned* out) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[65536 + 32768];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x * 16; i < 65536 + 32768; i += 64 * kWaves * 16)
    *reinterpret_cast<u32x4*>(lds + i) = u32x4{1u, 2u, 3u, (unsigned)i};
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, kSrcBytes, 0x00020000);
  // reads: the first 64 KB, rows 288 bytes apart, 16-byte groups per 16 lanes
  const unsigned rbase = (unsigned)((lane & 15) * 288 + (lane >> 4) * 16 + wave * 64);
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 held = acc;
  for (int it = 0; it < kSteps; ++it) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const unsigned a = (rbase + (unsigned)((it * 8 + u) & 7) * 4608u) & 65535u;
      acc ^= *reinterpret_cast<const u32x4*>(lds + (a & ~15u));
    }
    if (MODE != 0 && (it % STAGE) == 0) {
      // 1 KB per wave into the upper 32 KB (written, never read)
      const unsigned dst = 65536u + (unsigned)(((it / STAGE) * kWaves + wave) & 31) * 1024u;
      const unsigned off = (unsigned)(((blockIdx.x * 97 + it * 61 + wave) & 1023) * 1024 + 16 * lane);
      if (MODE == 1) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(lds + dst), 16, off, 0, 0, 0);
      } else if (MODE == 2) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(src + off);
        *reinterpret_cast<u32x4*>(lds + dst + 16 * lane) = x;
      } else {
        held ^= *reinterpret_cast<const u32x4*>(src + off);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  acc ^= held;
  if (acc.x + acc.y + acc.z + acc.w == 0x12345u) out[0] = 1;
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

unsigned char* g_src;
unsigned* g_out;
int g_cus;

template <int MODE, int STAGE>
void run(const char* what) {
  float t = time_ms([&] {
    hipLaunchKernelGGL((interfere<MODE, STAGE>), dim3(g_cus), dim3(64 * kWaves), 0, 0, g_src, g_out);
  });
  const double cyc = t * 1e-3 * 2.4e9;
  const double rd = (double)kWaves * kSteps * 8 * 1024;            // LDS read bytes per CU
  const double st = MODE ? (double)kWaves * (kSteps / STAGE) * 1024 : 0.0;  // staged bytes per CU
  printf("%-40s: %6.1f B/clk/CU of LDS reads, %5.1f B/clk/CU staged (%.3f ms)\n", what, rd / cyc, st / cyc, t);
}

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  g_cus = prop.multiProcessorCount;
  CHECK(hipMalloc(&g_src, kSrcBytes));
  CHECK(hipMemset(g_src, 1, kSrcBytes));
  CHECK(hipMalloc(&g_out, 64));
  printf("device %s, %d CUs, 16 waves per CU\n", prop.name, g_cus);
  run<0, 1>("reads only");
  run<1, 16>("+ direct load, 1 KB per 16 KB read");
  run<1, 8>("+ direct load, 1 KB per 8 KB read");
  run<1, 4>("+ direct load, 1 KB per 4 KB read");
  run<2, 16>("+ load + LDS store, 1 KB per 16 KB read");
  run<2, 8>("+ load + LDS store, 1 KB per 8 KB read");
  run<2, 4>("+ load + LDS store, 1 KB per 4 KB read");
  run<3, 16>("+ register load, 1 KB per 16 KB read");
  run<3, 8>("+ register load, 1 KB per 8 KB read");
  run<3, 4>("+ register load, 1 KB per 4 KB read");
  CHECK(hipFree(g_src));
  CHECK(hipFree(g_out));
  return 0;
}
