// Launchers of the backward kernels (bf16, d in {64, 128}, every N).
#include "attention_bwd.h"
#include "launch.h"

namespace tsa {

namespace {

template <int D, int N>
hipError_t launch_bwd_n(BwdParams p, long long bh, hipStream_t s) {
  p.n_qblocks = (p.L + DqCfg<D, N>::ROWS - 1) / DqCfg<D, N>::ROWS;
  const long long kblocks = bh * p.n_kblocks;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, N>), dim3((unsigned)kblocks), dim3(64 * DkdvCfg<D>::W), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long qblocks = bh * p.n_qblocks;
  hipLaunchKernelGGL((bwd_dq_kernel<D, N>), dim3((unsigned)qblocks), dim3(64 * DqCfg<D, N>::W), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, long long bh, int N, hipStream_t s) {
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)(bh * p.n_qc)), dim3(256), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (N) {
    case 1: return launch_bwd_n<D, 1>(p, bh, s);
    case 2: return launch_bwd_n<D, 2>(p, bh, s);
    case 4: return launch_bwd_n<D, 4>(p, bh, s);
    case 8: return launch_bwd_n<D, 8>(p, bh, s);
    case 16: return launch_bwd_n<D, 16>(p, bh, s);
    case 32: return launch_bwd_n<D, 32>(p, bh, s);
    case 64: return launch_bwd_n<D, 64>(p, bh, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attention_bwd(const BwdLaunch& a) {
  const tsa_problem_t* pr = a.p;
  BwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.dout = a.dout;
  p.lse = a.lse;
  p.mask = a.mask;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.ld = static_cast<float*>(a.workspace);
  p.L = pr->L;
  p.M = pr->M;
  p.T_q = (pr->L + pr->M - 1) / pr->M;
  const int T_k = (pr->L + pr->N - 1) / pr->N;
  p.words = (T_k + 31) / 32;
  p.n_qc = (pr->L + kBwdChunk - 1) / kBwdChunk;
  p.n_kblocks = (pr->L + DkdvCfg<128>::KEYS - 1) / DkdvCfg<128>::KEYS;
  p.n_qblocks = 0;  // set per N
  p.scale = a.scale;
  p.cs = fabsf(a.scale) * kLog2e;
  const long long bh = (long long)pr->B * pr->H;
  if (bh * p.n_qc > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  return pr->d == 128 ? launch_bwd_d<128>(p, bh, pr->N, a.stream) : launch_bwd_d<64>(p, bh, pr->N, a.stream);
}

}  // namespace tsa
