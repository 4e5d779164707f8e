// Quantisation of bf16 Q and K to FP8 (e4m3, OCP) with per-tile scales, the
// input of the FP8 attention path (gfx950).
//
// Q gets one scale per 16-row tile of a (b, h), K one per (b, h); a scale is
// (largest |x| of its tile) / 448 in float32, or 1 for an all-zero tile, so
// the largest value of a tile maps to 448, the largest e4m3 value.  Each
// value becomes the e4m3 number nearest to x / s (ties to even), from an
// IEEE float32 division and the hardware's round-to-nearest conversion.
// The passes read their input once and are bound by HBM bandwidth.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsa.h"
#include "tsa_device.h"

namespace tsa {

namespace {

constexpr int kD = 128;            // head dim of the FP8 path
constexpr float kE4m3Max = 448.f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// four floats / s -> four e4m3 bytes (little-endian in one word)
__device__ __forceinline__ uint32_t to_e4m3x4(float a, float b, float c, float d, float s) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a / s, b / s, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c / s, d / s, w, true);
  return (uint32_t)w;
}

// One wave per 16-row Q tile t: lane l takes row l/4, d = 32(l%4) .. +31.
__device__ __forceinline__ void quantize_q_tile(const bf16_t* __restrict__ q, int L, int t16, long long t,
                                                uint8_t* __restrict__ q8, float* __restrict__ q_scale) {
  const int lane = threadIdx.x & 63;
  const long long bh = t / t16;
  const int r = (int)(t - bh * t16) * 16 + (lane >> 2);
  const bool ok = r < L;
  const size_t off = ((size_t)bh * L + (ok ? r : 0)) * kD + 32 * (lane & 3);
  u32x4 x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    x[i] = ok ? *reinterpret_cast<const u32x4*>(q + off + 8 * i) : u32x4{0u, 0u, 0u, 0u};
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(fabsf(bf16_lo(x[i][e])), fabsf(bf16_hi(x[i][e]))));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float s = m > 0.f ? m / kE4m3Max : 1.f;
  if (lane == 0) q_scale[t] = s;
  if (!ok) return;
  u32x4 y[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[i >> 1][2 * (i & 1)] = to_e4m3x4(bf16_lo(x[i][0]), bf16_hi(x[i][0]), bf16_lo(x[i][1]), bf16_hi(x[i][1]), s);
    y[i >> 1][2 * (i & 1) + 1] =
        to_e4m3x4(bf16_lo(x[i][2]), bf16_hi(x[i][2]), bf16_lo(x[i][3]), bf16_hi(x[i][3]), s);
  }
  *reinterpret_cast<u32x4*>(q8 + off) = y[0];
  *reinterpret_cast<u32x4*>(q8 + off + 16) = y[1];
}

// Four tiles per work-group, stepping through the tiles with the grid's stride.
__global__ __launch_bounds__(256) void quantize_q_kernel(const bf16_t* __restrict__ q, int L, int t16,
                                                         long long tiles, uint8_t* __restrict__ q8,
                                                         float* __restrict__ q_scale) {
  for (long long tb = blockIdx.x; 4 * tb < tiles; tb += gridDim.x) {
    const long long t = 4 * tb + (threadIdx.x >> 6);
    if (t < tiles) quantize_q_tile(q, L, t16, t, q8, q_scale);
  }
}

// Largest |k| of each slice of a (b, h): unit u = (b*H + h) * S + slice
// writes the maximum of its slice to partial[u]; work-groups step through
// the units with the grid's stride.
constexpr int kKSlices = 64;  // slices per head (fewer for L < 2)

__global__ __launch_bounds__(256) void k_amax_kernel(const bf16_t* __restrict__ k, int L, int S, long long units,
                                                     float* __restrict__ partial) {
  __shared__ float part[4];
  for (long long u = blockIdx.x; u < units; u += gridDim.x) {
    const long long bh = u / S;
    const int slice = (int)(u - bh * S);
    const size_t n8 = (size_t)L * kD / 8;
    const size_t lo = n8 * slice / S, hi = n8 * (slice + 1) / S;
    const u32x4* kh = reinterpret_cast<const u32x4*>(k + (size_t)bh * L * kD);
    float m = 0.f;
    for (size_t i = lo + threadIdx.x; i < hi; i += 256) {
      const u32x4 x = kh[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(fabsf(bf16_lo(x[e])), fabsf(bf16_hi(x[e]))));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) partial[u] = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    __syncthreads();  // part is rewritten for the next unit
  }
}

// k_scale[b*H + h] from the head's partial maxima.
__global__ __launch_bounds__(256) void k_scale_kernel(const float* __restrict__ partial, int S, long long bh,
                                                      float* __restrict__ k_scale) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= bh) return;
  float m = 0.f;
  for (int s = 0; s < S; ++s) m = fmaxf(m, partial[i * S + s]);
  k_scale[i] = m > 0.f ? m / kE4m3Max : 1.f;
}

// K / its head's scale -> e4m3: eight values per thread.
__global__ __launch_bounds__(256) void quantize_k_kernel(const bf16_t* __restrict__ k, long long per_head8,
                                                         long long total8, const float* __restrict__ k_scale,
                                                         uint8_t* __restrict__ k8) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total8; i += (long long)gridDim.x * 256) {
    const float s = k_scale[i / per_head8];
    const u32x4 x = reinterpret_cast<const u32x4*>(k)[i];
    u32x2 y;
    y[0] = to_e4m3x4(bf16_lo(x[0]), bf16_hi(x[0]), bf16_lo(x[1]), bf16_hi(x[1]), s);
    y[1] = to_e4m3x4(bf16_lo(x[2]), bf16_hi(x[2]), bf16_lo(x[3]), bf16_hi(x[3]), s);
    reinterpret_cast<u32x2*>(k8)[i] = y;
  }
}

}  // namespace

hipError_t launch_quantize_qk_fp8(const tsa_problem_t* p, const void* q, const void* k, uint8_t* q8,
                                  float* q_scale, uint8_t* k8, float* k_scale, hipStream_t stream) {
  const long long bh = (long long)p->B * p->H;
  const int t16 = (p->L + 15) / 16;
  const long long tiles = bh * t16;
  hipLaunchKernelGGL(quantize_q_kernel, dim3(stride_blocks(tiles, 4)), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(q), p->L, t16, tiles, q8, q_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // The slice maxima go through k8 as scratch: B*H*S floats with S <= 32 L,
  // at most the B*H*L*128 bytes of k8, which quantize_k_kernel overwrites
  // only after k_scale_kernel has read them.
  const int S = p->L >= 2 ? kKSlices : 32;
  float* partial = reinterpret_cast<float*>(k8);
  hipLaunchKernelGGL(k_amax_kernel, dim3(stride_blocks(S * bh, 1)), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(k), p->L, S, S * bh, partial);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_scale_kernel, dim3((unsigned)((bh + 255) / 256)), dim3(256), 0, stream, partial, S, bh,
                     k_scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long long per_head8 = (long long)p->L * kD / 8;
  const long long total8 = bh * per_head8;
  hipLaunchKernelGGL(quantize_k_kernel, dim3(stride_blocks(total8, 256)), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(k), per_head8, total8, k_scale, k8);
  return hipGetLastError();
}

}  // namespace tsa
