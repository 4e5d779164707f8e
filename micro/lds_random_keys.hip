// LDS read rates of the N < 8 key kernel's operand patterns over random
// kept-key lists (Bernoulli keys of a 128-key chunk, density argv[1], default
// 0.2), for several row layouts of the staged K and V rows.
//   K: 8 ds_read_b128 per pass per lane; lane (g, n) reads key list[16b + n]
//      at bytes 16g + 64sl (score block b, d slab sl).
//   V: 16 ds_read_b64_tr_b16 per pass; lane (g, s) reads key
//      list[16h + 4g + (s >> 2)] at bytes 8(s & 3) + 32j (d block j).
// Layouts: 0 rows 288 bytes apart (the kernel's); 1, 2, 6 the same with the
// 16-byte pieces of a row permuted by bits of key >> 3; 3 rows 272 apart;
// 4, 5 rows 256 apart with pieces permuted by key & 15 or key >> 3; 7 rows
// 272 apart permuted by key >> 4.  Every offset is checked on the host
// against the LDS array, and each kernel exits after a fixed loop.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops micro/lds_random_keys.hip -o lds_random_keys
//   ./lds_random_keys 0.2 && ./lds_random_keys 1.0
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <vector>
#include <random>
#include <algorithm>
#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));              \
      exit(1);                                                                    \
    }                                                                             \
  } while (0)
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256, kIters = 2048, kLds = 128 * 288, NP = 512;
// offs: [NP][64 lanes][24]: 8 K offsets then 16 V offsets
__global__ __launch_bounds__(kThreads) void probe(const int* __restrict__ offs, int mode, unsigned* out) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
  for (int i = threadIdx.x; i < kLds / 4; i += kThreads) ((unsigned*)lds)[i] = i;
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int pat = (blockIdx.x * 4 + wv) % NP;
  int o[24];
  for (int i = 0; i < 24; ++i) o[i] = offs[(pat * 64 + lane) * 24 + i];
  u32x4 acc = {0, 0, 0, 0};
  i16x4 acv = {0, 0, 0, 0};
  for (int it = 0; it < kIters; ++it) {
    asm volatile("" ::: "memory");
    if (mode & 1) {
      u32x4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = *(const u32x4*)(lds + o[u]);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc ^= x[u];
    }
    if (mode & 2) {
      i16x4 y[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        y[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(lds + o[8 + u]));
#pragma unroll
      for (int u = 0; u < 16; ++u) acv ^= y[u];
    }
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w ^ (unsigned)acv.x ^ (unsigned)acv.w) == 0x12345u) out[0] = 1;
}
static int layout(int L, int key, int byte) {
  const int p = byte >> 4, r = byte & 15;
  switch (L) {
    case 0: return key * 288 + byte;
    case 1: return key * 288 + ((p ^ ((key >> 3) & 1)) << 4) + r;
    case 2: return key * 288 + ((p ^ ((key >> 3) & 3)) << 4) + r;
    case 3: return key * 272 + byte;
    case 4: return key * 256 + ((p ^ (key & 15)) << 4) + r;
    case 5: return key * 256 + ((p ^ ((key >> 3) & 15)) << 4) + r;
    case 6: return key * 288 + ((p ^ ((key >> 3) & 7)) << 4) + r;
    default: return key * 272 + ((p ^ ((key >> 4) & 3)) << 4) + r;
  }
}
int main(int argc, char** argv) {
  const double dens = argc > 1 ? atof(argv[1]) : 0.2;
  hipDeviceProp_t pr;
  CHECK(hipGetDeviceProperties(&pr, 0));
  const int cus = pr.multiProcessorCount; const double clk = pr.clockRate * 1e3;
  std::mt19937 rng(12345);
  std::vector<std::vector<int>> lists(NP);
  for (auto& l : lists) {
    std::vector<int> keys;
    for (int k = 0; k < 128; ++k) if (std::uniform_real_distribution<double>(0, 1)(rng) < dens) keys.push_back(k);
    if (keys.empty()) keys.push_back(0);
    l.assign(32, keys[0]);
    for (int i = 0; i < 32 && i < (int)keys.size(); ++i) l[i] = keys[i];
  }
  int* d;
  unsigned* out;
  CHECK(hipMalloc(&d, NP * 64 * 24 * 4));
  CHECK(hipMalloc(&out, 4));
  const int blocks = cus * 8;
  printf("density %.2f\n", dens);
  for (int L = 0; L < 8; ++L) {
    std::vector<int> h(NP * 64 * 24);
    for (int pt = 0; pt < NP; ++pt)
      for (int lane = 0; lane < 64; ++lane) {
        const int g = lane >> 4, n = lane & 15, s = n;
        int* o = &h[(pt * 64 + lane) * 24];
        for (int b = 0; b < 2; ++b) for (int sl = 0; sl < 4; ++sl)
          o[b * 4 + sl] = layout(L, lists[pt][16 * b + n], 16 * g + 64 * sl);
        for (int hh = 0; hh < 2; ++hh) for (int j = 0; j < 8; ++j)
          o[8 + hh * 8 + j] = layout(L, lists[pt][16 * hh + 4 * g + (s >> 2)], 8 * (s & 3) + 32 * j);
        for (int i = 0; i < 24; ++i) {
          const int w = i < 8 ? 16 : 8;
          if (o[i] < 0 || o[i] + w > kLds || o[i] % w) { fprintf(stderr, "bad offset L%d\n", L); return 1; }
        }
      }
    CHECK(hipMemcpy(d, h.data(), h.size() * 4, hipMemcpyHostToDevice));
    for (int mode = 1; mode <= 3; ++mode) {
      hipEvent_t a, b;
      CHECK(hipEventCreate(&a));
      CHECK(hipEventCreate(&b));
      hipLaunchKernelGGL(probe, dim3(blocks), dim3(kThreads), 0, 0, d, mode, out);
      CHECK(hipDeviceSynchronize());
      CHECK(hipEventRecord(a));
      for (int r = 0; r < 3; ++r) hipLaunchKernelGGL(probe, dim3(blocks), dim3(kThreads), 0, 0, d, mode, out);
      CHECK(hipEventRecord(b));
      CHECK(hipEventSynchronize(b));
      float ms;
      CHECK(hipEventElapsedTime(&ms, a, b));
      ms /= 3;
      const double bytes = (double)blocks * kThreads * kIters * ((mode & 1 ? 8 * 16 : 0) + (mode & 2 ? 16 * 8 : 0));
      printf("layout %d mode %s %7.1f B/clk/CU\n", L, mode == 1 ? "K   " : mode == 2 ? "V   " : "K+V ", bytes / (ms * 1e-3) / clk / cus);
    }
  }
  return 0;
}
