// Host-side validation and partitioning (pure C++, no HIP calls).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "attn_decode.h"

namespace attn {

constexpr int kChunkQuantum = 64;        // a forced chunk_len must be a multiple of this
constexpr int kChunkGrain = 256;         // automatic chunk lengths are multiples of this
constexpr int kMaxValuRows = 8;          // rows per VALU work item
constexpr int kMfmaRows = 32;            // rows per MFMA work item
constexpr int kMaxRows = 1 << 16;        // G * q_len limit
// Work items per CU.  Dense calls (every sequence full) use one contiguous
// chunk per CU: each CU streams one long run of K/V, which measured fastest
// on MI355X.  With device-side ragged lengths the host cannot balance
// exactly, so chunks are made finer and items past a sequence's end exit.
constexpr int kDenseItemsPerCu = 1;
constexpr int kRaggedItemsPerCu = 4;

int items_per_cu(bool ragged);
attn_status_t validate_desc(const attn_desc_t *d);
attn_status_t make_plan(const attn_desc_t *d, int cu_count, bool mfma_available, attn_plan_t *p);
size_t partial_bytes(int64_t records, int head_dim);
attn_status_t validate_bifurcated(const attn_bifurcated_desc_t *d);
void bifurcated_descs(const attn_bifurcated_desc_t *d, attn_desc_t *prefix, attn_desc_t *suffix);

}  // namespace attn
