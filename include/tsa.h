/*
 * tsa.h - fine-grained tile-sparse softmax attention (forward and backward) for AMD MI355X (gfx950).
 *
 * The operation is the one described in the abstract of "FG-Attn: Leveraging
 * Fine-Grained Sparse Attention in Video Diffusion Models" (section Abstract):
 * the attention score matrix of each (batch, head) is cut into tiles of M
 * queries by N keys (M >= 16, N >= 1); a tile is either computed or skipped as
 * a whole, and skipped scores take no part in the softmax.
 *
 * Conventions shared by every call:
 *   - Q, K, V, O are contiguous row-major [B][H][L][d] device arrays of one
 *     element type (fp32 or bf16); d is innermost.
 *   - The keep-bitmap is a contiguous uint32 device array [B][H][T_q][W] with
 *     T_q = ceil(L/M), T_k = ceil(L/N), W = ceil(T_k/32).  Key tile j of query
 *     tile i is bit (j % 32) of word (j / 32) of row (b, h, i), least significant
 *     bit first; 1 keeps the tile.  Bits at j >= T_k are padding and ignored.
 *   - The last query tile and the last key tile may be partial (L need not be a
 *     multiple of M or N); rows and keys at index >= L do not exist.
 *   - A query row with no kept key gets O = 0 and LSE = -inf.
 *   - Every call is asynchronous on the caller's `stream` (a hipStream_t; NULL
 *     is the default stream).  Outputs are valid once the stream has reached
 *     the work.  The library allocates no device memory and the caller owns
 *     every buffer.  Between calls it keeps only the calling thread's
 *     measurement events (tsa_set_timing_events), the last error text, and
 *     the static per-GPU scratch of tsa_attention_fwd_noalloc.
 *   - Arguments are checked before anything is enqueued.  A failed check
 *     enqueues nothing and returns a status; no call aborts or throws.
 *     tsa_last_error() returns the calling thread's detail text of its last
 *     failure.
 *
 * Supported problem set: dtype in {F32, BF16}; d in {64, 128}; M in {16, 32, 64};
 * N in {1, 2, 4, 8, 16, 32, 64}; 1 <= L <= 2^22; B*H <= 2^20; and for the
 * attention calls B*H*(L + 256) <= 2^30 - 1 (their grids hold about 4
 * work-items per row; any problem whose tensors fit in device memory
 * qualifies).  Other values return TSA_ERR_UNSUPPORTED.
 */
#ifndef TSA_H_
#define TSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TSA_OK = 0,
  TSA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, non-positive size, bad scale, ... */
  TSA_ERR_UNSUPPORTED = 2,        /* (dtype, d, M, N) outside the supported set */
  TSA_ERR_WORKSPACE_TOO_SMALL = 3,
  TSA_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} tsa_status_t;

typedef enum { TSA_DTYPE_F32 = 0, TSA_DTYPE_BF16 = 1 } tsa_dtype_t;

typedef enum {
  TSA_OP_ATTENTION_FWD = 0,
  TSA_OP_MASK_COMPACT = 1,
  TSA_OP_PREDICT_MASK = 2,
  TSA_OP_ATTENTION_BWD = 3
} tsa_op_t;

/* Problem shape: batch B, heads H, sequence length L, head dim d, tile M x N. */
typedef struct {
  int32_t B, H, L, d, M, N;
  tsa_dtype_t dtype;
} tsa_problem_t;

/* Number of uint32 words per bitmap row, ceil(ceil(L/N)/32); 0 if L or N < 1.
 * Host only. */
int64_t tsa_mask_row_words(int32_t L, int32_t N);

/* Device workspace in bytes that `op` needs for problem `p` (may be 0).  Host
 * only; enqueues nothing. */
tsa_status_t tsa_workspace_size(tsa_op_t op, const tsa_problem_t* p, size_t* bytes);

/* Tile-sparse attention forward (FG-Attn abstract: scores skipped per M x N
 * tile, skipped scores excluded from the softmax):
 *   O[b,h,r,:] = sum_c P[r,c] V[b,h,c,:],  P[r,:] = softmax over kept c of
 *   scale * Q[b,h,r,:] . K[b,h,c,:], where c is kept iff bit(b,h,r/M,c/N) = 1.
 * q, k, v: [B,H,L,d] of p->dtype.  mask_bits: [B,H,T_q,W] uint32.
 * o: [B,H,L,d] of p->dtype, written for every row (must not alias q, k, v).
 * lse: optional [B,H,L] fp32 natural-log sum-exp of the kept scaled scores
 * (NULL skips it).  scale: finite.  Accumulation is fp32; bf16 inputs are
 * multiplied on bf16 matrix cores with the probabilities rounded to bf16.
 * workspace: tsa_workspace_size(TSA_OP_ATTENTION_FWD) bytes, 256-byte aligned;
 * the call packs V transposed into it (B*H*(d+1)*ceil(L/128)*128 elements)
 * and, for bf16 with N >= 8 and L <= 262144, writes after it (at the next
 * 256-byte boundary) a 64-word bitmap of the 128-key chunks each group of
 * 256 query rows keeps a tile of, one flag word per group and a count of
 * flagged groups, before the attention kernels read them.  Its contents are not needed after the call
 * returns control of the stream. */
tsa_status_t tsa_attention_fwd(const tsa_problem_t* p,
                               const void* q, const void* k, const void* v,
                               const uint32_t* mask_bits, float scale,
                               void* o, float* lse,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/* tsa_attention_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments, layouts, results and errors
 * are those of tsa_attention_fwd; the workspace it would take
 * (tsa_workspace_size(TSA_OP_ATTENTION_FWD)) lives instead in a static device
 * array of 64 MiB that the library holds on every GPU it runs on until the
 * process ends.  A problem that needs more (at d = 128, bf16: about
 * B*H*L > 250 000, e.g. 5 heads at L = 32760 fit) returns
 * TSA_ERR_UNSUPPORTED and enqueues nothing.  The call allocates nothing:
 * the array's device address is looked up once per device, with that device
 * current, on the first call.  The GPU is the current device, which must be
 * the stream's.  All calls on one GPU share the array: calls that overlap on
 * one GPU (other streams, other threads) race and give wrong results;
 * calls ordered on one stream are safe, and every call rewrites all of the
 * scratch it reads. */
tsa_status_t tsa_attention_fwd_noalloc(const tsa_problem_t* p,
                                       const void* q, const void* k, const void* v,
                                       const uint32_t* mask_bits, float scale,
                                       void* o, float* lse, void* stream);

/* Measurement hook: the forward calls made afterwards by this thread
 * (tsa_attention_fwd, tsa_attention_fwd_noalloc, tsa_attention_fwd_fp8)
 * record start_event on their stream right before the attention kernel(s)
 * proper and stop_event right after them, so that hipEventElapsedTime gives the
 * kernels' time without the V^T pack and the chunk pre-pass that the call
 * also enqueues.  Both are hipEvent_t handles created by the caller, passed
 * as void*; NULL, NULL switches recording off (the default).  Giving only one
 * returns TSA_ERR_INVALID_ARGUMENT.  The events must outlive the calls that
 * record them. */
tsa_status_t tsa_set_timing_events(void* start_event, void* stop_event);

/* FP8 inputs of tsa_attention_fwd_fp8: q and k (bf16 [B,H,L,128]) as e4m3
 * bytes (OCP format: 4 exponent bits, bias 7, 3 mantissa bits, largest value
 * 448) with per-tile scales: q_scale [B,H,ceil(L/16)] fp32, one per 16-row tile
 * of a head, and k_scale [B,H] fp32, one per head.  A scale is the tile's
 * largest |x| / 448 (1 for an all-zero tile); a value becomes the e4m3 number
 * nearest to x / scale, ties to even.  q8, k8: [B,H,L,128] bytes.  p->dtype must
 * be bf16 and p->d 128; M and N are not read.  No workspace
 * (k8 serves as scratch for the per-head maxima before it is written).  The quantisation
 * is this library's reading of the per-tile scaling named beside the pages'
 * method (FG-Attn itself fixes no precision). */
tsa_status_t tsa_quantize_qk_fp8(const tsa_problem_t* p, const void* q, const void* k,
                                 uint8_t* q8, float* q_scale, uint8_t* k8, float* k_scale,
                                 void* stream);

/* tsa_attention_fwd with FP8 scores (FG-Attn abstract: scores skipped per
 * M x N tile, skipped scores excluded from the softmax): the scores are
 * scale * (q8 . k8) * q_scale[tile of r] * k_scale[head], computed on the
 * 16x16x128 FP8 matrix cores; V, the probabilities and O are bf16 as in
 * tsa_attention_fwd.  q8, k8, q_scale, k_scale as tsa_quantize_qk_fp8 writes
 * them; v, mask_bits, o, lse, scale and the workspace
 * (tsa_workspace_size(TSA_OP_ATTENTION_FWD)) as in tsa_attention_fwd.
 * Supported: p->dtype bf16, d = 128, M in {16, 32, 64}, N in
 * {1, 2, 4, 8, 16, 32, 64}; other shapes return TSA_ERR_UNSUPPORTED. */
tsa_status_t tsa_attention_fwd_fp8(const tsa_problem_t* p,
                                   const uint8_t* q8, const uint8_t* k8,
                                   const float* q_scale, const float* k_scale,
                                   const void* v, const uint32_t* mask_bits, float scale,
                                   void* o, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Gradients of tsa_attention_fwd's output with respect to q, k and v, for an
 * upstream gradient d_o.  The pages define only the forward (FG-Attn abstract:
 * skipped M x N tiles excluded from the softmax); this is its derivative by the
 * chain rule, with P the forward's kept-score softmax and
 * D[r] = sum_d d_o[r,d] o[r,d]:
 *   dv = P^T d_o,  dS = P * (d_o v^T - D),  dq = scale dS k,  dk = scale dS^T q.
 * Skipped tiles get no work; a query row with no kept key contributes nothing.
 * q, k, v, o, d_o: [B,H,L,d] bf16 (o is the forward's output).  lse: [B,H,L]
 * fp32, the forward's log-sum-exp (required; -inf marks a row with no kept
 * key).  mask_bits and scale: as passed to the forward.  dq, dk, dv: [B,H,L,d]
 * bf16, written in full, none aliasing an input.  Accumulation is fp32; the
 * probabilities and dS are rounded to bf16 for the matrix cores.
 * workspace: tsa_workspace_size(TSA_OP_ATTENTION_BWD) bytes, 256-byte aligned
 * (B*H*ceil(L/128)*256 floats: per 128-row chunk the rows' LSE*log2(e) and D);
 * not needed after the call.  Supported: bf16 with the forward's d, M and N;
 * fp32 returns TSA_ERR_UNSUPPORTED. */
tsa_status_t tsa_attention_bwd(const tsa_problem_t* p,
                               const void* q, const void* k, const void* v,
                               const void* o, const void* d_o, const float* lse,
                               const uint32_t* mask_bits, float scale,
                               void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/* Difference of two keep-bitmaps of problem p, for reusing a predicted mask
 * across denoising steps (FG-Attn abstract: one keep decision per M x N tile):
 * row_changed[(b*H + h)*T_q + i] = number of key tiles j < T_k whose keep bit
 * differs between mask_a and mask_b in row (b, h, i) (padding bits ignored);
 * head_changed[b*H + h] = the sum over the head's rows (NULL skips it).
 * mask_a, mask_b: [B,H,T_q,W] uint32 device arrays (read only; they may be
 * the same).  row_changed: [B*H*T_q] int64, head_changed: [B*H] int64, device,
 * written in full, 8-byte aligned.  No workspace; d and dtype are not read. */
tsa_status_t tsa_mask_diff(const tsa_problem_t* p, const uint32_t* mask_a, const uint32_t* mask_b,
                           int64_t* row_changed, int64_t* head_changed, void* stream);

/* Mask compaction (FG-Attn abstract: one skip decision per M x N tile): every
 * bitmap row (b,h,i) becomes the ascending list of its kept key tiles j < T_k.
 * row_ptr: [B*H*T_q + 1] int64, rows in (b,h,i) row-major order, row_ptr[0]=0,
 * always written in full.  col_idx: int32 key-tile indices; entries at
 * positions >= col_capacity are not written, so the caller checks
 * row_ptr[B*H*T_q] <= col_capacity.  p->d, p->dtype are ignored.
 * workspace: tsa_workspace_size(TSA_OP_MASK_COMPACT) bytes. */
tsa_status_t tsa_mask_compact(const tsa_problem_t* p, const uint32_t* mask_bits,
                              int64_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Tile-mask predictor from pooled queries and keys.  The FG-Attn abstract
 * takes the tile mask as an input; this call produces one: Qbar_i = mean of
 * the (valid) rows of query tile i, Kbar_j = mean of the keys of key tile j,
 * s_ij = Qbar_i . Kbar_j in fp32, and row i keeps its
 * k = T_k - 1 - floor(sparsity_percent * (T_k - 1) / 100) highest-scoring
 * tiles, equal scores going to the smaller j.  With distinct scores these are
 * the tiles strictly above the row's linearly interpolated
 * sparsity_percent-th percentile.  q, k: [B,H,L,d]; 0 <= sparsity_percent < 100.
 * mask_out: [B,H,T_q,W] uint32, written in full (padding bits zero).
 * No score is stored: the workspace holds the pooled means and a list of
 * rows for an exact per-row pass.
 * workspace: tsa_workspace_size(TSA_OP_PREDICT_MASK) bytes. */
tsa_status_t tsa_predict_mask(const tsa_problem_t* p, const void* q, const void* k,
                              int32_t sparsity_percent, uint32_t* mask_out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* tsa_status_string(tsa_status_t s);

/* Detail text of the calling thread's last failed call ("" if none). */
const char* tsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TSA_H_ */
