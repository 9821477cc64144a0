/*
 * attn_decode_testing.h -- test-only views of the work partition and of the
 * argument checks.
 *
 * Not part of the decode boundary, and not exported by libattn_decode.so:
 * these functions live in the test build of the library
 * (libattn_decode_testing.so, which also exports everything attn_decode.h
 * declares).  The partition functions run on the host the same arithmetic
 * the kernels run on the device (how the KV segments of a call are cut into
 * per-workgroup pieces and where each piece's record goes), with the
 * sequence lengths given as a host array; they and the check functions make
 * no HIP call, and cu_count must be positive.  The library keeps no state
 * that these functions could change.
 */
#ifndef ATTN_DECODE_TESTING_H
#define ATTN_DECODE_TESTING_H

#include <stddef.h>
#include <stdint.h>

#include "attn_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Pieces of workgroup w: writes up to max_pieces entries of four int64
 * (segment, first token, end token, record slot) to out and returns the
 * number of pieces (a negative attn_status_t on invalid arguments).
 * host_lens: int32[batch] or NULL (every sequence max_kv_len long). */
ATTN_API int64_t attn_testing_pieces(const attn_desc_t *desc, const int32_t *host_lens,
                                     int32_t cu_count, int64_t w, int64_t *out,
                                     int64_t max_pieces);

/* Record slots of segment `segment`: out = {first, stride, count}. */
ATTN_API attn_status_t attn_testing_segment_slots(const attn_desc_t *desc,
                                                  const int32_t *host_lens, int32_t cu_count,
                                                  int64_t segment, int64_t out[3]);

/* Whether attn_prefill_anchor takes its single-merge path for this shape on
 * cu_count CUs: 1 when every segment of both the anchor part and the local
 * part is a single piece (the local split then merges each row's two
 * records itself and no merge launch follows), 0 otherwise, or a negative
 * attn_status_t on invalid arguments. */
ATTN_API int32_t attn_testing_anchor_fuses(const attn_anchor_desc_t *desc, int32_t cu_count);

/* The partitioner's plan for cu_count (>= 1) CUs, as attn_decode_plan. */
ATTN_API attn_status_t attn_testing_plan(const attn_desc_t *desc, int32_t cu_count,
                                         attn_plan_t *plan);

/* The host checks of the decode entry points on their own: tensor pointers
 * (need_v: V is read; need_o: O is written), outputs and the paging
 * description (NULL: dense).  Returns what the entry point would. */
ATTN_API attn_status_t attn_testing_check_decode(const attn_desc_t *desc,
                                                 const attn_paged_kv_t *paged, const void *q,
                                                 const void *k, const void *v, const float *o,
                                                 const float *lse, int32_t need_v,
                                                 int32_t need_o);

/* The host checks and workspace size of attn_decode_bifurcated for cu_count
 * CUs. */
ATTN_API attn_status_t attn_testing_check_bifurcated(const attn_bifurcated_desc_t *desc,
                                                     int32_t cu_count, size_t *workspace_bytes);

/* How attn_decode_bifurcated would launch on cu_count CUs: *prefix_wgs and
 * *suffix_wgs are the workgroup counts of the two parts' work maps.  One
 * launch of both parts: their sum is cu_count when the CUs are split between
 * them, both are cu_count when every workgroup takes a share of both; two
 * separate split launches: *fused = 0. */
ATTN_API attn_status_t attn_testing_bifurcated_form(const attn_bifurcated_desc_t *desc,
                                                   int32_t cu_count, int32_t *fused,
                                                   int64_t *prefix_wgs, int64_t *suffix_wgs);

/* attn_prefill_anchor always on its three-launch path (anchor split, local
 * split, merge), whatever the shape; arguments, results and errors as
 * attn_prefill_anchor.  For comparing the two paths in tests. */
ATTN_API attn_status_t attn_testing_prefill_anchor_unfused(
    const attn_anchor_desc_t *desc, const void *q, const void *k_anchor, const void *v_anchor,
    const void *k_blocks, const void *v_blocks, float *o, float *lse, void *workspace,
    size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_DECODE_TESTING_H */
