// C ABI of the tile-sparse attention library: argument validation, workspace
// sizing, dispatch to the kernel launchers, and error reporting.  Nothing is
// enqueued unless every check passes; no exception or abort crosses the ABI.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.h"
#include "tsa.h"
#include "tsa_workload.h"

namespace tsa {
hipError_t launch_mask_compact(const tsa_problem_t* p, const uint32_t* mask, int64_t* row_ptr,
                               int32_t* col_idx, int64_t col_capacity, void* workspace,
                               hipStream_t stream);
size_t mask_compact_workspace(const tsa_problem_t* p);
hipError_t launch_predict_mask(const tsa_problem_t* p, const void* q, const void* k,
                               int sparsity_percent, uint32_t* mask_out, void* workspace,
                               hipStream_t stream);
size_t predict_workspace(const tsa_problem_t* p);
hipError_t launch_maskgen_structured(const tsa_problem_t* p, const tsa_structured_params_t* s,
                                     const int32_t* head_pattern, uint32_t* out, hipStream_t stream);
hipError_t launch_maskgen_hash(const tsa_problem_t* p, const tsa_maskgen_params_t* g,
                               uint32_t* out, hipStream_t stream);
hipError_t launch_mask_diff(const tsa_problem_t* p, const uint32_t* a, const uint32_t* b, int64_t* rows_out,
                            int64_t* heads_out, hipStream_t stream);
}  // namespace tsa

namespace {

thread_local char g_err[512] = "";
// events of tsa_set_timing_events, used by the forward calls of this thread
thread_local hipEvent_t g_ev_start = nullptr;
thread_local hipEvent_t g_ev_stop = nullptr;

tsa_status_t fail(tsa_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

tsa_status_t hip_fail(hipError_t e, const char* what) {
  return fail(TSA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

constexpr int kMaxL = 1 << 22;
constexpr long long kMaxBH = 1 << 20;
// A dispatch holds fewer than 2^32 work-items in each grid dimension.  The
// attention kernels' grids hold at most 4 work-items per (b, h) and key (or
// query) row, padding included; every other kernel steps through its items
// with a capped grid.
constexpr long long kMaxWorkItems = 0xffffffffLL;
inline bool attention_grid_fits(const tsa_problem_t* p) {
  return (long long)p->B * p->H * ((long long)p->L + 256) * 4 <= kMaxWorkItems;
}

// Shape checks common to every call.  need_d: check d and dtype.
tsa_status_t check_problem(const tsa_problem_t* p, bool need_d) {
  if (p == nullptr) return fail(TSA_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->B < 1 || p->H < 1 || p->L < 1 || p->M < 1 || p->N < 1 || (need_d && p->d < 1))
    return fail(TSA_ERR_INVALID_ARGUMENT, "sizes must be positive (B=%d H=%d L=%d d=%d M=%d N=%d)",
                p->B, p->H, p->L, p->d, p->M, p->N);
  if (p->L > kMaxL) return fail(TSA_ERR_UNSUPPORTED, "L=%d exceeds %d", p->L, kMaxL);
  if ((long long)p->B * p->H > kMaxBH)
    return fail(TSA_ERR_UNSUPPORTED, "B*H=%lld exceeds %lld", (long long)p->B * p->H, kMaxBH);
  if (!(p->M == 16 || p->M == 32 || p->M == 64))
    return fail(TSA_ERR_UNSUPPORTED, "M=%d not in {16, 32, 64}", p->M);
  if (!pow2_in(p->N, 1, 64))
    return fail(TSA_ERR_UNSUPPORTED, "N=%d not in {1, 2, 4, 8, 16, 32, 64}", p->N);
  if (need_d) {
    if (!(p->d == 64 || p->d == 128)) return fail(TSA_ERR_UNSUPPORTED, "d=%d not in {64, 128}", p->d);
    if (!(p->dtype == TSA_DTYPE_F32 || p->dtype == TSA_DTYPE_BF16))
      return fail(TSA_ERR_UNSUPPORTED, "dtype=%d not supported", (int)p->dtype);
  }
  return TSA_OK;
}

// Argument checks of the forward, shared by its two entry points.
tsa_status_t check_fwd(const tsa_problem_t* p, const void* q, const void* k, const void* v,
                       const uint32_t* mask_bits, float scale, const void* o, const float* lse) {
  tsa_status_t s = check_problem(p, true);
  if (s != TSA_OK) return s;
  if (!q || !k || !v || !mask_bits || !o)
    return fail(TSA_ERR_INVALID_ARGUMENT, "q, k, v, mask_bits and o must be non-NULL");
  if (!std::isfinite(scale)) return fail(TSA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(mask_bits, 4) || (lse && !aligned(lse, 4)))
    return fail(TSA_ERR_INVALID_ARGUMENT, "q/k/v/o need 16-byte, mask/lse 4-byte alignment");
  if (o == q || o == k || o == v) return fail(TSA_ERR_INVALID_ARGUMENT, "o aliases an input");
  if (!attention_grid_fits(p)) return fail(TSA_ERR_UNSUPPORTED, "B*H*(L+256) above 2^30: grid too large");
  return TSA_OK;
}

tsa_status_t launch_fwd(const tsa_problem_t* p, const void* q, const void* k, const void* v,
                        const uint32_t* mask_bits, float scale, void* o, float* lse, void* workspace,
                        void* stream) {
  tsa::AttnLaunch a{p, q, k, v, mask_bits, scale, o, lse, workspace, static_cast<hipStream_t>(stream)};
  a.ev_start = g_ev_start;
  a.ev_stop = g_ev_stop;
  const hipError_t e = p->dtype == TSA_DTYPE_BF16 ? tsa::launch_attention_bf16(a)
                                                  : tsa::launch_attention_f32(a);
  if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  return TSA_OK;
}

// Scratch of tsa_attention_fwd_noalloc: the forward's workspace (packed V^T
// and the chunk-skip words) for callers that cannot allocate.  Every GPU the
// library runs on holds its own copy until the process ends; calls on one GPU
// share it.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's copy of `scratch`, looked up once per device
// with that device current (the array's name is not a device address in host
// code).
tsa_status_t scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(TSA_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr || !aligned(ptr, 256)) return fail(TSA_ERR_HIP, "scratch has no usable address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TSA_OK;
}

}  // namespace

extern "C" {

int64_t tsa_mask_row_words(int32_t L, int32_t N) {
  if (L < 1 || N < 1) return 0;
  const int64_t T_k = ((int64_t)L + N - 1) / N;
  return (T_k + 31) / 32;
}

tsa_status_t tsa_workspace_size(tsa_op_t op, const tsa_problem_t* p, size_t* bytes) {
  if (bytes == nullptr) return fail(TSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  tsa_status_t s;
  switch (op) {
    case TSA_OP_ATTENTION_FWD:
      if ((s = check_problem(p, true)) != TSA_OK) return s;
      *bytes = tsa::attention_workspace_bytes(p);
      return TSA_OK;
    case TSA_OP_MASK_COMPACT:
      if ((s = check_problem(p, false)) != TSA_OK) return s;
      *bytes = tsa::mask_compact_workspace(p);
      return TSA_OK;
    case TSA_OP_PREDICT_MASK:
      if ((s = check_problem(p, true)) != TSA_OK) return s;
      *bytes = tsa::predict_workspace(p);
      return TSA_OK;
    case TSA_OP_ATTENTION_BWD:
      if ((s = check_problem(p, true)) != TSA_OK) return s;
      if (p->dtype != TSA_DTYPE_BF16) return fail(TSA_ERR_UNSUPPORTED, "backward supports bf16 only");
      *bytes = tsa::attention_bwd_workspace_bytes(p);
      return TSA_OK;
  }
  return fail(TSA_ERR_INVALID_ARGUMENT, "unknown op %d", (int)op);
}

tsa_status_t tsa_attention_fwd(const tsa_problem_t* p, const void* q, const void* k, const void* v,
                               const uint32_t* mask_bits, float scale, void* o, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream) {
  tsa_status_t s = check_fwd(p, q, k, v, mask_bits, scale, o, lse);
  if (s != TSA_OK) return s;
  const size_t need = tsa::attention_workspace_bytes(p);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(TSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, 256-byte aligned (got %zu)",
                need, workspace_bytes);
  return launch_fwd(p, q, k, v, mask_bits, scale, o, lse, workspace, stream);
}

tsa_status_t tsa_attention_fwd_noalloc(const tsa_problem_t* p, const void* q, const void* k,
                                       const void* v, const uint32_t* mask_bits, float scale, void* o,
                                       float* lse, void* stream) {
  tsa_status_t s = check_fwd(p, q, k, v, mask_bits, scale, o, lse);
  if (s != TSA_OK) return s;
  const size_t need = tsa::attention_workspace_bytes(p);
  if (need > kScratchBytes)
    return fail(TSA_ERR_UNSUPPORTED,
                "problem needs %zu bytes of scratch; tsa_attention_fwd_noalloc holds at most %zu "
                "(call tsa_attention_fwd with a workspace instead)", need, kScratchBytes);
  void* ws = nullptr;
  if ((s = scratch_for_current_device(&ws)) != TSA_OK) return s;
  return launch_fwd(p, q, k, v, mask_bits, scale, o, lse, ws, stream);
}

tsa_status_t tsa_quantize_qk_fp8(const tsa_problem_t* p, const void* q, const void* k, uint8_t* q8,
                                 float* q_scale, uint8_t* k8, float* k_scale, void* stream) {
  tsa_status_t s = check_problem(p, true);
  if (s != TSA_OK) return s;
  if (p->dtype != TSA_DTYPE_BF16 || p->d != 128)
    return fail(TSA_ERR_UNSUPPORTED, "FP8 quantisation takes bf16 q, k with d = 128");
  if (!q || !k || !q8 || !q_scale || !k8 || !k_scale)
    return fail(TSA_ERR_INVALID_ARGUMENT, "q, k, q8, q_scale, k8 and k_scale must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(q8, 16) || !aligned(k8, 16) || !aligned(q_scale, 4) ||
      !aligned(k_scale, 4))
    return fail(TSA_ERR_INVALID_ARGUMENT, "tensors need 16-byte, scales 4-byte alignment");
  const hipError_t e = tsa::launch_quantize_qk_fp8(p, q, k, q8, q_scale, k8, k_scale,
                                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "FP8 quantisation launch");
  return TSA_OK;
}

tsa_status_t tsa_attention_fwd_fp8(const tsa_problem_t* p, const uint8_t* q8, const uint8_t* k8,
                                   const float* q_scale, const float* k_scale, const void* v,
                                   const uint32_t* mask_bits, float scale, void* o, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  tsa_status_t s = check_problem(p, true);
  if (s != TSA_OK) return s;
  if (p->dtype != TSA_DTYPE_BF16 || p->d != 128)
    return fail(TSA_ERR_UNSUPPORTED, "FP8 attention: bf16 v/o and d = 128 (got d=%d)", p->d);
  if (!q8 || !k8 || !q_scale || !k_scale || !v || !mask_bits || !o)
    return fail(TSA_ERR_INVALID_ARGUMENT, "q8, k8, q_scale, k_scale, v, mask_bits and o must be non-NULL");
  if (!std::isfinite(scale)) return fail(TSA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(mask_bits, 4) ||
      !aligned(q_scale, 4) || !aligned(k_scale, 4) || (lse && !aligned(lse, 4)))
    return fail(TSA_ERR_INVALID_ARGUMENT, "q8/k8/v/o need 16-byte, mask/scales/lse 4-byte alignment");
  if (o == v || o == (const void*)q8 || o == (const void*)k8)
    return fail(TSA_ERR_INVALID_ARGUMENT, "o aliases an input");
  const size_t need = tsa::attention_workspace_bytes(p);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(TSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, 256-byte aligned (got %zu)",
                need, workspace_bytes);
  if (!attention_grid_fits(p)) return fail(TSA_ERR_UNSUPPORTED, "B*H*(L+256) above 2^30: grid too large");
  tsa::AttnLaunch a{p, q8, k8, v, mask_bits, scale, o, lse, workspace, static_cast<hipStream_t>(stream)};
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.ev_start = g_ev_start;
  a.ev_stop = g_ev_stop;
  const hipError_t e = tsa::launch_attention_fp8(a);
  if (e != hipSuccess) return hip_fail(e, "FP8 attention kernel launch");
  return TSA_OK;
}

tsa_status_t tsa_attention_bwd(const tsa_problem_t* p, const void* q, const void* k, const void* v,
                               const void* o, const void* d_o, const float* lse,
                               const uint32_t* mask_bits, float scale, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, void* stream) {
  tsa_status_t s = check_problem(p, true);
  if (s != TSA_OK) return s;
  if (p->dtype != TSA_DTYPE_BF16) return fail(TSA_ERR_UNSUPPORTED, "backward supports bf16 only");
  if (!q || !k || !v || !o || !d_o || !lse || !mask_bits || !dq || !dk || !dv)
    return fail(TSA_ERR_INVALID_ARGUMENT, "q, k, v, o, d_o, lse, mask_bits, dq, dk and dv must be non-NULL");
  if (!std::isfinite(scale)) return fail(TSA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(d_o, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(mask_bits, 4) ||
      !aligned(lse, 4))
    return fail(TSA_ERR_INVALID_ARGUMENT, "tensors need 16-byte, mask/lse 4-byte alignment");
  const void* ins[] = {q, k, v, o, d_o, lse};
  for (const void* x : ins)
    if (x == dq || x == dk || x == dv) return fail(TSA_ERR_INVALID_ARGUMENT, "a gradient aliases an input");
  if (dq == dk || dq == dv || dk == dv) return fail(TSA_ERR_INVALID_ARGUMENT, "gradients alias each other");
  const size_t need = tsa::attention_bwd_workspace_bytes(p);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(TSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, 256-byte aligned (got %zu)",
                need, workspace_bytes);
  if (!attention_grid_fits(p)) return fail(TSA_ERR_UNSUPPORTED, "B*H*(L+256) above 2^30: grid too large");
  tsa::BwdLaunch a{p, q, k, v, o, d_o, lse, mask_bits, scale, dq, dk, dv, workspace,
                   static_cast<hipStream_t>(stream)};
  const hipError_t e = tsa::launch_attention_bwd(a);
  if (e != hipSuccess) return hip_fail(e, "backward kernel launch");
  return TSA_OK;
}

tsa_status_t tsa_mask_diff(const tsa_problem_t* p, const uint32_t* mask_a, const uint32_t* mask_b,
                           int64_t* row_changed, int64_t* head_changed, void* stream) {
  tsa_status_t s = check_problem(p, false);
  if (s != TSA_OK) return s;
  if (!mask_a || !mask_b || !row_changed)
    return fail(TSA_ERR_INVALID_ARGUMENT, "mask_a, mask_b and row_changed must be non-NULL");
  if (!aligned(mask_a, 4) || !aligned(mask_b, 4) || !aligned(row_changed, 8) ||
      (head_changed && !aligned(head_changed, 8)))
    return fail(TSA_ERR_INVALID_ARGUMENT, "masks need 4-byte, counts 8-byte alignment");
  const hipError_t e = tsa::launch_mask_diff(p, mask_a, mask_b, row_changed, head_changed,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mask diff launch");
  return TSA_OK;
}

tsa_status_t tsa_mask_compact(const tsa_problem_t* p, const uint32_t* mask_bits, int64_t* row_ptr,
                              int32_t* col_idx, int64_t col_capacity, void* workspace,
                              size_t workspace_bytes, void* stream) {
  tsa_status_t s = check_problem(p, false);
  if (s != TSA_OK) return s;
  if (!mask_bits || !row_ptr) return fail(TSA_ERR_INVALID_ARGUMENT, "mask_bits and row_ptr must be non-NULL");
  if (col_capacity < 0) return fail(TSA_ERR_INVALID_ARGUMENT, "col_capacity < 0");
  if (col_capacity > 0 && !col_idx) return fail(TSA_ERR_INVALID_ARGUMENT, "col_idx is NULL");
  if (!aligned(mask_bits, 4) || !aligned(row_ptr, 8) || (col_idx && !aligned(col_idx, 4)))
    return fail(TSA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  const size_t need = tsa::mask_compact_workspace(p);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(TSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, 256-byte aligned (got %zu)",
                need, workspace_bytes);
  const hipError_t e = tsa::launch_mask_compact(p, mask_bits, row_ptr, col_idx, col_capacity,
                                                 workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "compaction kernel launch");
  return TSA_OK;
}

tsa_status_t tsa_predict_mask(const tsa_problem_t* p, const void* q, const void* k,
                              int32_t sparsity_percent, uint32_t* mask_out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  tsa_status_t s = check_problem(p, true);
  if (s != TSA_OK) return s;
  if (!q || !k || !mask_out) return fail(TSA_ERR_INVALID_ARGUMENT, "q, k and mask_out must be non-NULL");
  if (sparsity_percent < 0 || sparsity_percent >= 100)
    return fail(TSA_ERR_INVALID_ARGUMENT, "sparsity_percent=%d outside [0, 100)", sparsity_percent);
  if (!aligned(q, 4) || !aligned(k, 4) || !aligned(mask_out, 4))
    return fail(TSA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  const size_t need = tsa::predict_workspace(p);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(TSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, 256-byte aligned (got %zu)",
                need, workspace_bytes);
  const hipError_t e = tsa::launch_predict_mask(p, q, k, sparsity_percent, mask_out, workspace,
                                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "predictor kernel launch");
  return TSA_OK;
}

tsa_status_t tsa_maskgen_hash(const tsa_problem_t* p, const tsa_maskgen_params_t* g,
                              uint32_t* mask_out, void* stream) {
  tsa_status_t s = check_problem(p, false);
  if (s != TSA_OK) return s;
  if (!g || !mask_out) return fail(TSA_ERR_INVALID_ARGUMENT, "params and mask_out must be non-NULL");
  if (g->frame_tokens < 0 || g->frame_radius < 0 || g->thr_near > (1u << 24) || g->thr_far > (1u << 24))
    return fail(TSA_ERR_INVALID_ARGUMENT, "bad generator parameters");
  const hipError_t e = tsa::launch_maskgen_hash(p, g, mask_out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mask generator launch");
  return TSA_OK;
}

tsa_status_t tsa_maskgen_structured(const tsa_problem_t* p, const tsa_structured_params_t* g,
                                    const int32_t* head_pattern, uint32_t* mask_out, void* stream) {
  tsa_status_t s = check_problem(p, false);
  if (s != TSA_OK) return s;
  if (!g || !head_pattern || !mask_out)
    return fail(TSA_ERR_INVALID_ARGUMENT, "params, head_pattern and mask_out must be non-NULL");
  if (p->H > TSA_MAX_PATTERN_HEADS)
    return fail(TSA_ERR_UNSUPPORTED, "at most %d heads", TSA_MAX_PATTERN_HEADS);
  bool multi = false, stripe = false;
  for (int h = 0; h < p->H; ++h) {
    const int32_t t = head_pattern[h];
    if (t < TSA_PATTERN_EMPTY || t > TSA_PATTERN_DENSE)
      return fail(TSA_ERR_INVALID_ARGUMENT, "head %d: unknown pattern %d", h, (int)t);
    multi = multi || t == TSA_PATTERN_MULTI_DIAGONAL;
    stripe = stripe || t == TSA_PATTERN_VERTICAL_STRIPE;
  }
  if (g->diag_width < 0 || g->band_width < 0 ||
      (multi && (g->frame_tokens <= 0 || g->reach < 0 || g->reach > 64)) ||
      (stripe && (g->stripe_period <= 0 || g->stripe_width < 0 || g->stripe_width > g->stripe_period)))
    return fail(TSA_ERR_INVALID_ARGUMENT, "bad structured-mask parameters");
  const hipError_t e = tsa::launch_maskgen_structured(p, g, head_pattern, mask_out,
                                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mask generator launch");
  return TSA_OK;
}

tsa_status_t tsa_set_timing_events(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(TSA_ERR_INVALID_ARGUMENT, "give both events or neither");
  g_ev_start = static_cast<hipEvent_t>(start_event);
  g_ev_stop = static_cast<hipEvent_t>(stop_event);
  return TSA_OK;
}

const char* tsa_status_string(tsa_status_t s) {
  switch (s) {
    case TSA_OK: return "success";
    case TSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case TSA_ERR_UNSUPPORTED: return "unsupported problem";
    case TSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case TSA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* tsa_last_error(void) { return g_err; }

}  // extern "C"
