// Host-side validation and partitioning (pure C++, no HIP calls).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "attn_decode.h"
#include "kv_paging.h"
#include "work_map.h"

namespace attn {

constexpr int kChunkQuantum = 64;        // a forced chunk_len must be a multiple of this
constexpr int kMinPiece = 256;           // balanced layout: tokens per workgroup, at least
constexpr int kMaxValuRows = 8;          // rows per VALU work item
constexpr int kMfmaRows = 32;            // rows per MFMA work item
constexpr int kMaxRows = 1 << 16;        // G * q_len limit
constexpr int64_t kMaxUnits = int64_t(1) << 46;  // B * Hkv * row_blocks * max_kv_len limit
// Workgroups per CU in the balanced layout: one contiguous share of the
// tokens per CU, which measured fastest on MI355X (each CU streams one long
// run of K/V).
constexpr int kItemsPerCu = 1;
// Tokens per CU below which the vector-ALU kernel gets twice the workgroups.
constexpr int64_t kShortShare = 2048;

int items_per_cu(int kernel, int64_t units, int cu_count);
attn_status_t validate_desc(const attn_desc_t *d);
// Host checks of a paging description against its descriptor (null paged:
// dense caches, always valid).  Fills *pg for the kernels.
constexpr int kMaxPageShift = 20;
attn_status_t validate_paged(const attn_desc_t *d, const attn_paged_kv_t *paged, KvPaging *pg);
// Addressing of a dense [B][Hkv][L_max][D] cache.
KvPaging dense_paging(const attn_desc_t *d);
attn_status_t make_plan(const attn_desc_t *d, int cu_count, bool mfma_available, attn_plan_t *p);
size_t partial_bytes(int64_t records, int head_dim);
WorkMap work_map(const attn_desc_t *d, const attn_plan_t &p);
attn_status_t validate_bifurcated(const attn_bifurcated_desc_t *d);
void bifurcated_descs(const attn_bifurcated_desc_t *d, attn_desc_t *prefix, attn_desc_t *suffix);
attn_status_t validate_anchor(const attn_anchor_desc_t *d);
void anchor_descs(const attn_anchor_desc_t *d, attn_desc_t *anchor, attn_desc_t *local);

}  // namespace attn
