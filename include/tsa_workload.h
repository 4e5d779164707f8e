/*
 * tsa_workload.h - synthetic keep-bitmap generator (workload support).
 *
 * Not part of the attention method: it produces seeded (and structured) test
 * and benchmark masks on the GPU for sizes whose bitmaps are too large to draw on the host
 * (e.g. 40 heads x 4725 x 75600 tiles).  It implements the same counter-based
 * generator as the host-side workload package, bit for bit:
 *
 *   ctr = ((b*H + h)*T_q + i)*T_k + j
 *   z   = SplitMix64 output number ctr+1 of a stream whose state starts at
 *         state0 (Steele, Lea & Flood, "Fast splittable pseudorandom number
 *         generators", OOPSLA 2014: state += 0x9E3779B97F4A7C15, then the
 *         mix (z^(z>>30))*0xBF58476D1CE4E5B9, (z^(z>>27))*0x94D049BB133111EB,
 *         z^(z>>31))
 *   keep(b,h,i,j) = (z >> 40) < thr, thr = thr_near when
 *         |floor(i*M/frame_tokens) - floor(j*N/frame_tokens)| <= frame_radius
 *         (or frame_tokens == 0), else thr_far;
 *   and, if force_diag, every tile whose key range [jN, jN+N) overlaps the
 *   query tile's rows [iM, iM+M) (both clipped to L) is kept.
 *
 * Output bitmap layout is that of tsa.h; padding bits are written as 0.
 */
#ifndef TSA_WORKLOAD_H_
#define TSA_WORKLOAD_H_

#include <stdint.h>

#include "tsa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  uint64_t state0;      /* SplitMix64 starting state */
  uint32_t thr_near;    /* 24-bit keep thresholds, round(p * 2^24) */
  uint32_t thr_far;
  int32_t frame_tokens; /* 0: no frame structure */
  int32_t frame_radius;
  int32_t force_diag;   /* nonzero: keep tiles overlapping the diagonal */
} tsa_maskgen_params_t;

/* Writes mask_out [B,H,T_q,W] for problem p (p->d and p->dtype ignored). */
tsa_status_t tsa_maskgen_hash(const tsa_problem_t* p, const tsa_maskgen_params_t* g,
                              uint32_t* mask_out, void* stream);

/*
 * Structured keep-bitmaps, one pattern per head.  The patterns are the three
 * recurring structures of video-DiT attention maps named by "Sparse-vDiT:
 * Unleashing the Power of Sparse Attention to Accelerate Video Diffusion
 * Transformers" (abstract: diagonal, multi-diagonal, vertical-stripe, and
 * heads that can be skipped entirely); the token-level rules below are this
 * library's reading of those names.  A tile (i, j) is kept iff the rule
 * holds for at least one query row q in [iM, min(iM+M, L)) and key k in
 * [jN, min(jN+N, L)):
 *   EMPTY:           never (the head is skipped; its output rows are zero)
 *   DIAGONAL:        |q - k| <= diag_width
 *   MULTI_DIAGONAL:  |q - k - t*frame_tokens| <= band_width for some
 *                    integer t, |t| <= reach (a band repeated every frame)
 *   VERTICAL_STRIPE: (k mod stripe_period) < stripe_width (the same key
 *                    columns for every query)
 *   DENSE:           always
 */
typedef enum {
  TSA_PATTERN_EMPTY = 0,
  TSA_PATTERN_DIAGONAL = 1,
  TSA_PATTERN_MULTI_DIAGONAL = 2,
  TSA_PATTERN_VERTICAL_STRIPE = 3,
  TSA_PATTERN_DENSE = 4
} tsa_pattern_t;

#define TSA_MAX_PATTERN_HEADS 128

typedef struct {
  int32_t diag_width;     /* DIAGONAL half-width in tokens, >= 0 */
  int32_t band_width;     /* MULTI_DIAGONAL band half-width in tokens, >= 0 */
  int32_t frame_tokens;   /* MULTI_DIAGONAL spacing, > 0 when that pattern is used */
  int32_t reach;          /* MULTI_DIAGONAL: 0 <= reach <= 64 */
  int32_t stripe_period;  /* VERTICAL_STRIPE period, > 0 when that pattern is used */
  int32_t stripe_width;   /* 0 <= stripe_width <= stripe_period */
} tsa_structured_params_t;

/* Writes mask_out [B,H,T_q,W] for problem p (p->d and p->dtype ignored);
 * head_pattern: host array of H tsa_pattern_t values (H <=
 * TSA_MAX_PATTERN_HEADS), the same for every batch index.  Padding bits are
 * written as 0.  Errors: INVALID_ARGUMENT for a bad pattern or parameter,
 * UNSUPPORTED for H > TSA_MAX_PATTERN_HEADS. */
tsa_status_t tsa_maskgen_structured(const tsa_problem_t* p, const tsa_structured_params_t* s,
                                    const int32_t* head_pattern, uint32_t* mask_out,
                                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TSA_WORKLOAD_H_ */
