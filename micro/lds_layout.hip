// LDS layout probe for the attention kernel's operand reads (gfx950).
//
// Each case is a table of 64 per-lane byte offsets into a 32 KB LDS block;
// every wave of the grid reads 16 (or 8) bytes at its lane's offset eight
// times per iteration.  The rate reached (bytes per clock per CU) shows how
// many bank conflicts the layout costs: row strides and octet pairings of
// the K-row and V^T-column reads are compared.  All offsets are in bounds
// (checked on the host) and every kernel exits after a fixed loop.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops micro/lds_layout.hip -o lds_layout
//   ./lds_layout
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

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

constexpr int kThreads = 256;
constexpr int kIters = 2048;
constexpr int kLds = 65536;

// Read u of an iteration goes to offs[lane] + u * step: step 0 re-reads one
// address, other steps move the whole pattern (to test whether address bits
// above the pattern's own change the bank mapping).
template <int W>
__global__ __launch_bounds__(kThreads) void probe(const int* __restrict__ offs, int step,
                                                  unsigned* out) {
  __shared__ __attribute__((aligned(16))) unsigned lds[kLds / 4];
  for (int i = threadIdx.x; i < kLds / 4; i += kThreads) lds[i] = i;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const char* p = reinterpret_cast<const char*>(lds) + offs[lane];
  for (int it = 0; it < kIters; ++it) {
    if constexpr (W == 16) {
      u32x4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        asm volatile("" ::: "memory");
        x[u] = *reinterpret_cast<const u32x4*>(p + u * step);
      }
      asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]),
                   "v"(x[7]));
    } else {
      u32x2 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        asm volatile("" ::: "memory");
        x[u] = *reinterpret_cast<const u32x2*>(p + u * step);
      }
      asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]),
                   "v"(x[7]));
    }
  }
  if (lane == 64) out[0] = 1;
}

struct Case {
  std::string name;
  int w;
  std::vector<int> off;
};

// K rows of a 16-key score block: lane (g, n) reads row 8*oct[n>>3] + (n&7)
// at byte 16*g of the row (one 32-element d slab).
static Case k_rows(int stride, int o0, int o1) {
  Case c{"K rows, stride " + std::to_string(stride) + ", octets " + std::to_string(o0) + "," +
             std::to_string(o1),
         16, std::vector<int>(64)};
  for (int l = 0; l < 64; ++l) {
    const int g = l >> 4, n = l & 15;
    const int row = 8 * (n < 8 ? o0 : o1) + (n & 7);
    c.off[l] = row * stride + 16 * g;
  }
  return c;
}

// K rows of the four-octet layout: row 8*oct[n>>2] + (n&3).
static Case k_rows4(int stride, int a, int b, int cc, int d) {
  const int o[4] = {a, b, cc, d};
  Case c{"K rows x4, stride " + std::to_string(stride) + ", octets " + std::to_string(a) + "," +
             std::to_string(b) + "," + std::to_string(cc) + "," + std::to_string(d),
         16, std::vector<int>(64)};
  for (int l = 0; l < 64; ++l) {
    const int g = l >> 4, n = l & 15;
    c.off[l] = (8 * o[n >> 2] + (n & 3)) * stride + 16 * g;
  }
  return c;
}

// V^T columns, 16 bytes: lane (g, n) reads row n at octet column oct[g].
static Case vt_b128(int stride, int a, int b, int cc, int d) {
  const int o[4] = {a, b, cc, d};
  Case c{"V^T b128, stride " + std::to_string(stride) + ", octets " + std::to_string(a) + "," +
             std::to_string(b) + "," + std::to_string(cc) + "," + std::to_string(d),
         16, std::vector<int>(64)};
  for (int l = 0; l < 64; ++l) c.off[l] = (l & 15) * stride + 16 * o[l >> 4];
  return c;
}

// V^T columns, 8 bytes: lane (g, n) reads row n at half (g&1) of octet oct[g>>1].
static Case vt_b64(int stride, int a, int b) {
  Case c{"V^T b64, stride " + std::to_string(stride) + ", octets " + std::to_string(a) + "," +
             std::to_string(b),
         8, std::vector<int>(64)};
  for (int l = 0; l < 64; ++l) {
    const int g = l >> 4, n = l & 15;
    c.off[l] = n * stride + 16 * (g < 2 ? a : b) + 8 * (g & 1);
  }
  return c;
}

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  const double clk = 2.4e9;
  std::vector<Case> cases;
  for (int st : {136, 144, 152, 176}) {
    cases.push_back(vt_b64(st, 0, 1));
    cases.push_back(vt_b64(st, 5, 2));
  }
  for (int st : {160, 176}) {
    cases.push_back(k_rows(st, 0, 1));
    cases.push_back(k_rows(st, 3, 6));
  }
  for (int st : {272, 288}) {
    cases.push_back(k_rows(st, 0, 1));
    cases.push_back(k_rows(st, 2, 7));
    cases.push_back(k_rows(st, 0, 2));
    cases.push_back(k_rows4(st, 0, 1, 2, 3));
    cases.push_back(k_rows4(st, 1, 5, 6, 10));
    cases.push_back(vt_b128(st, 0, 1, 2, 3));
    cases.push_back(vt_b128(st, 3, 7, 10, 15));
    cases.push_back(vt_b64(st, 0, 1));
    cases.push_back(vt_b64(st, 5, 9));
  }
  int* d_off;
  unsigned* out;
  CHECK(hipMalloc(&d_off, 64 * sizeof(int)));
  CHECK(hipMalloc(&out, 64));
  const int blocks = cus * 8;
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  printf("device %s, %d CUs\n", prop.name, cus);
  for (const Case& c : cases)
  for (int mode = 0; mode < 4; ++mode) {
    const int stride = std::stoi(c.name.substr(c.name.find("stride ") + 7));
    const int step = mode == 0 ? 0 : mode == 1 ? 4096 : mode == 2 ? 16 * stride : 256;
    for (int l = 0; l < 64; ++l) {
      if (c.off[l] < 0 || c.off[l] + 7 * step + c.w > kLds || c.off[l] % c.w != 0) {
        fprintf(stderr, "case %s: lane %d offset %d out of range\n", c.name.c_str(), l, c.off[l]);
        return 1;
      }
    }
    CHECK(hipMemcpy(d_off, c.off.data(), 64 * sizeof(int), hipMemcpyHostToDevice));
    auto launch = [&] {
      if (c.w == 16) hipLaunchKernelGGL(probe<16>, dim3(blocks), dim3(kThreads), 0, 0, d_off, step, out);
      else hipLaunchKernelGGL(probe<8>, dim3(blocks), dim3(kThreads), 0, 0, d_off, step, out);
    };
    launch();
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(a));
    for (int r = 0; r < 3; ++r) launch();
    CHECK(hipEventRecord(b));
    CHECK(hipEventSynchronize(b));
    float ms;
    CHECK(hipEventElapsedTime(&ms, a, b));
    ms /= 3;
    const double bytes = (double)blocks * kThreads * c.w * 8.0 * kIters;
    printf("%-44s step %5d %7.1f B/clk/CU\n", c.name.c_str(), step, bytes / (ms * 1e-3) / clk / cus);
  }
  CHECK(hipFree(d_off));
  CHECK(hipFree(out));
  return 0;
}
