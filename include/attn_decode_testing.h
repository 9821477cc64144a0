/*
 * attn_decode_testing.h -- host-side views of the work partition, for tests.
 *
 * Not part of the decode boundary.  These run on the host the same
 * partition arithmetic the kernels run on the device (how the KV segments of
 * a call are cut into per-workgroup pieces and where each piece's record
 * goes), with the sequence lengths given as a host array.  No HIP call is
 * made; cu_count must be positive.
 */
#ifndef ATTN_DECODE_TESTING_H
#define ATTN_DECODE_TESTING_H

#include <stdint.h>

#include "attn_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Pieces of workgroup w: writes up to max_pieces entries of four int64
 * (segment, first token, end token, record slot) to out and returns the
 * number of pieces (a negative attn_status_t on invalid arguments).
 * host_lens: int32[batch] or NULL (every sequence max_kv_len long). */
int64_t attn_testing_pieces(const attn_desc_t *desc, const int32_t *host_lens, int32_t cu_count,
                            int64_t w, int64_t *out, int64_t max_pieces);

/* Record slots of segment `segment`: out = {first, stride, count}. */
attn_status_t attn_testing_segment_slots(const attn_desc_t *desc, const int32_t *host_lens,
                                         int32_t cu_count, int64_t segment, int64_t out[3]);

/* Whether attn_prefill_anchor takes its finalising path for this shape on
 * cu_count CUs: 1 when every segment of both the anchor part and the local
 * part is a single piece (the local split then merges each row's two
 * records itself and no merge launch follows), 0 otherwise, or a negative
 * attn_status_t on invalid arguments. */
int32_t attn_testing_anchor_fuses(const attn_anchor_desc_t *desc, int32_t cu_count);

/* enabled = 0 makes attn_prefill_anchor always take the unfused path
 * (anchor split, local split, merge), 1 restores the default.  Process-wide;
 * for comparing the two paths in tests. */
void attn_testing_set_anchor_fusion(int32_t enabled);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_DECODE_TESTING_H */
