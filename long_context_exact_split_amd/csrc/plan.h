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
// Largest token extent of a KV cache (max_kv_len, prefix, suffix and anchor
// lengths).  The kernels index tokens in 32-bit arithmetic and compute token
// indices up to a few hundred tokens past the last one they use before
// clamping them, so the extent stays 2^16 below 2^31.
constexpr int64_t kMaxKvLen = (int64_t(1) << 31) - (int64_t(1) << 16);
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
// mfma_available: dense query blocks may take the matrix-core kernels.
attn_status_t make_plan(const attn_desc_t *d, int cu_count, bool mfma_available, attn_plan_t *p);
size_t partial_bytes(int64_t records, int head_dim);
WorkMap work_map(const attn_desc_t *d, const attn_plan_t &p);
attn_status_t validate_bifurcated(const attn_bifurcated_desc_t *d);
void bifurcated_descs(const attn_bifurcated_desc_t *d, attn_desc_t *prefix, attn_desc_t *suffix);
attn_status_t validate_anchor(const attn_anchor_desc_t *d);
void anchor_descs(const attn_anchor_desc_t *d, attn_desc_t *anchor, attn_desc_t *local);

// Argument checks of the decode entry points that need no device: null
// tensors (allowed where they would hold no element), base alignment
// (16 bytes for inputs, 4 for the fp32 outputs) and the workspace.
bool aligned(const void *p, uintptr_t a);
attn_status_t check_inputs(const attn_desc_t *d, const void *q, const void *k, const void *v,
                           bool need_v);
attn_status_t check_outputs(const attn_desc_t *d, const float *o, const float *lse, bool need_o);
attn_status_t check_workspace(size_t need, const void *ws, size_t ws_bytes);

// The shared-prefix call as two decode calls (prefix: one sequence whose
// query tokens are the samples; suffix: one token per sample) and their
// plans; the suffix records follow the prefix records in the workspace.
// fused: both splits run in one launch of `workgroups` workgroups (the
// prefix on the shared-tile kernel in 256-row blocks, the suffix on the
// vector-ALU code), each plan rebalanced over that many workgroups.
struct BifPlans {
  attn_desc_t pre, suf;
  attn_plan_t pp, sp;
  size_t pre_bytes, total;
  bool fused;
  int64_t workgroups;
};
// A balanced plan re-cut over W workgroups (the record slots and workspace
// follow).
attn_status_t set_workgroups(const attn_desc_t *d, int64_t W, attn_plan_t *p);
attn_status_t bifurcated_plans(const attn_bifurcated_desc_t *d, int cu, BifPlans *b);

// The anchor-block prefill as two calls over the same rows: the anchor part
// (one cache shared by every block) and the causal local part.  fuse: the
// local split merges each row's two records itself (every segment of both
// parts is one piece of the shared-tile kernel, with the same row blocks),
// so no merge launch follows; allow_fusion = false always takes the
// three-launch path.
struct AnchorPlans {
  attn_desc_t anc, loc;
  attn_plan_t ap, lp;
  size_t anc_bytes, total;
  bool fuse;
};
attn_status_t anchor_plans(const attn_anchor_desc_t *d, int cu, bool allow_fusion,
                           AnchorPlans *a);
// True when every segment of a balanced layout is a single piece.
bool whole_segment_pieces(const WorkMap &m);

}  // namespace attn
