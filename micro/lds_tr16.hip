// LDS read rate of the PV operand pattern of the octet kernel (gfx950) read
// two ways: transposing reads of V rows (ds_read_b64_tr_b16) and plain 8-byte
// reads.  Lane group g reads keys 4(g&1)..4(g&1)+3 of octet o_(g>>1) of a
// 16-octet chunk; lane s of a group points at row s>>2, d = 4(s&3).. of it.
// Every access stays inside the kernel's LDS array and each kernel exits
// after a fixed number of iterations.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops micro/lds_tr16.hip -o lds_tr16
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
constexpr int kThreads = 256, kIters = 4096;
template <int STRIDE>
__global__ __launch_bounds__(kThreads) void tr_oct(unsigned* out, int oa, int ob) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[16 * 8 * STRIDE];  // 16 octets
  for (int i = threadIdx.x; i < 16 * 8 * STRIDE / 4; i += kThreads) ((unsigned*)lds)[i] = i;
  __syncthreads();
  const int lane = threadIdx.x & 63, g = lane >> 4, s = lane & 15;
  const int wv = threadIdx.x >> 6;
  const int oct = (g >> 1) ? ob : oa;
  const int row = 8 * oct + 4 * (g & 1) + (s >> 2);
  const unsigned char* p = lds + row * STRIDE + 8 * (s & 3);
  i16x4 acc = {0, 0, 0, 0};
  for (int it = 0; it < kIters / 8; ++it) {
    asm volatile("" ::: "memory");
    i16x4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      x[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(p + 32 * ((u + it + wv) & 7)));
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= x[u];
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x1234) out[0] = 1;
}
template <int STRIDE>
__global__ __launch_bounds__(kThreads) void b64_oct(unsigned* out, int oa, int ob) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[16 * 8 * STRIDE];
  for (int i = threadIdx.x; i < 16 * 8 * STRIDE / 4; i += kThreads) ((unsigned*)lds)[i] = i;
  __syncthreads();
  const int lane = threadIdx.x & 63, g = lane >> 4, s = lane & 15;
  const int wv = threadIdx.x >> 6;
  const int oct = (g >> 1) ? ob : oa;
  const int row = 8 * oct + 4 * (g & 1) + (s >> 2);
  const unsigned char* p = lds + row * STRIDE + 8 * (s & 3);
  u32x2 acc = {0, 0};
  for (int it = 0; it < kIters / 8; ++it) {
    asm volatile("" ::: "memory");
    u32x2 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = *(const u32x2*)(p + 32 * ((u + it + wv) & 7));
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= x[u];
  }
  if ((acc.x ^ acc.y) == 0x1234) out[0] = 1;
}
template <typename F> float time_ms(F f) {
  hipEvent_t a, b; hipEventCreate(&a); hipEventCreate(&b);
  f(); hipDeviceSynchronize(); hipEventRecord(a);
  for (int r = 0; r < 5; ++r) f();
  hipEventRecord(b); hipEventSynchronize(b); float ms; hipEventElapsedTime(&ms, a, b); return ms / 5;
}
int main() {
  hipDeviceProp_t pr; hipGetDeviceProperties(&pr, 0);
  const int cus = pr.multiProcessorCount; const double clk = pr.clockRate * 1e3;
  unsigned* out; hipMalloc(&out, 4);
  const int blocks = cus * 8;
  const double bytes = (double)blocks * kThreads * 8 * kIters;
  auto rep = [&](const char* w, float ms) { printf("%-40s %7.1f B/clk/CU (%.3f ms)\n", w, bytes / (ms * 1e-3) / clk / cus, ms); };
  int pairs[3][2] = {{0, 1}, {5, 2}, {3, 12}};
  for (auto& q : pairs) {
    char nm[64];
    snprintf(nm, 64, "tr16 stride 288 octets %d,%d", q[0], q[1]);
    rep(nm, time_ms([&] { hipLaunchKernelGGL(tr_oct<288>, dim3(blocks), dim3(kThreads), 0, 0, out, q[0], q[1]); }));
    snprintf(nm, 64, "tr16 stride 272 octets %d,%d", q[0], q[1]);
    rep(nm, time_ms([&] { hipLaunchKernelGGL(tr_oct<272>, dim3(blocks), dim3(kThreads), 0, 0, out, q[0], q[1]); }));
    snprintf(nm, 64, "b64  stride 288 octets %d,%d", q[0], q[1]);
    rep(nm, time_ms([&] { hipLaunchKernelGGL(b64_oct<288>, dim3(blocks), dim3(kThreads), 0, 0, out, q[0], q[1]); }));
  }
  printf("clock %.0f MHz\n", clk / 1e6);
  return 0;
}
