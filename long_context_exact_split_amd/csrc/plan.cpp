// Host-side validation and KV-chunk partitioning (no HIP calls).
//
// The partitioner turns one decode call into work items (b, KV head, row
// block, chunk).  Tree Attention computes one local energy per device and
// Star Attention one block per host; on one GPU the unit of parallel work is
// the workgroup, so the chunk length C is chosen so that the number of items
// is a small multiple of the compute-unit count: every CU streams about the
// same number of KV bytes, and the per-chunk records stay a tiny fraction of
// the KV traffic.
#include "plan.h"

#include <cmath>
#include <cstdlib>
#include <limits>

namespace attn {
namespace {

int env_int(const char *name, int fallback, int lo, int hi) {
  const char *s = std::getenv(name);
  if (!s || !*s) return fallback;
  char *end = nullptr;
  long v = std::strtol(s, &end, 10);
  if (end == s || v < lo || v > hi) return fallback;
  return (int)v;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

int items_per_cu(bool ragged) {
  static const int forced = env_int("ATTN_DECODE_ITEMS_PER_CU", 0, 1, 1024);
  if (forced > 0) return forced;
  return ragged ? kRaggedItemsPerCu : kDenseItemsPerCu;
}

attn_status_t validate_desc(const attn_desc_t *d) {
  if (!d) return ATTN_ERR_NULL;
  if (d->dtype != ATTN_BF16 && d->dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (d->batch < 0 || d->q_len < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
      d->num_q_heads % d->num_kv_heads != 0 || d->max_kv_len < 0 ||
      d->max_kv_len > std::numeric_limits<int32_t>::max() || d->head_dim < 1)
    return ATTN_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(d->scale)) return ATTN_ERR_VALUE;
  if (d->causal != 0 && d->causal != 1) return ATTN_ERR_VALUE;
  if (d->chunk_len < 0 || d->chunk_len % kChunkQuantum != 0) return ATTN_ERR_VALUE;
  const int64_t R = (int64_t)(d->num_q_heads / d->num_kv_heads) * d->q_len;
  if (R > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

attn_status_t make_plan(const attn_desc_t *d, int cu_count, bool mfma_available, attn_plan_t *p) {
  attn_status_t st = validate_desc(d);
  if (st != ATTN_OK) return st;
  if (!p) return ATTN_ERR_NULL;
  if (cu_count < 1) return ATTN_ERR_VALUE;
  const int G = d->num_q_heads / d->num_kv_heads;
  const int R = G * d->q_len;
  *p = attn_plan_t{};
  p->rows = R;
  p->cu_count = cu_count;
  p->threads_per_item = 256;
  // Dense query blocks (many rows per KV head) go to the MFMA kernel; a few
  // rows per KV head are a bandwidth-bound stream for the vector ALUs.
  p->kernel = (mfma_available && d->dtype == ATTN_BF16 && R > kMaxValuRows) ? 1 : 0;
  if (p->kernel == 0) {
    p->rows_per_block = R <= 1 ? 1 : R <= 2 ? 2 : R <= 4 ? 4 : 8;
  } else {
    p->rows_per_block = kMfmaRows;
  }
  p->row_blocks = (R + p->rows_per_block - 1) / p->rows_per_block;
  const int64_t groups = (int64_t)d->batch * d->num_kv_heads;
  const int64_t L = d->max_kv_len;
  int64_t C;
  if (d->chunk_len > 0) {
    C = d->chunk_len;
  } else {
    const int64_t work = groups * p->row_blocks * L;
    const int64_t target = (int64_t)cu_count * items_per_cu(d->kv_lens != nullptr);
    C = round_up((work + target - 1) / (target > 0 ? target : 1), kChunkGrain);
    if (C < kChunkGrain) C = kChunkGrain;
    const int64_t whole = round_up(L > 0 ? L : 1, kChunkGrain);
    if (C > whole) C = whole;
  }
  if (C > std::numeric_limits<int32_t>::max()) return ATTN_ERR_UNSUPPORTED;
  p->chunk_len = (int32_t)C;
  const int64_t chunks = L > 0 ? (L + C - 1) / C : 0;
  p->chunks_per_seq = (int32_t)chunks;
  p->work_items = groups * p->row_blocks * chunks;
  if (p->work_items > std::numeric_limits<int32_t>::max()) return ATTN_ERR_UNSUPPORTED;
  const int64_t records = groups * chunks * (int64_t)p->row_blocks * p->rows_per_block;
  p->workspace_bytes = partial_bytes(records, d->head_dim);
  return ATTN_OK;
}

size_t partial_bytes(int64_t records, int head_dim) {
  if (records <= 0) return 0;
  const size_t ml = (size_t)round_up(records * (int64_t)sizeof(float), 256);
  const size_t o = (size_t)round_up(records * (int64_t)head_dim * (int64_t)sizeof(float), 256);
  return 2 * ml + o;
}

attn_status_t validate_bifurcated(const attn_bifurcated_desc_t *d) {
  if (!d) return ATTN_ERR_NULL;
  if (d->dtype != ATTN_BF16) return d->dtype == ATTN_F32 ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_DTYPE;
  if (d->num_samples < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
      d->num_q_heads % d->num_kv_heads != 0 || d->prefix_len < 0 || d->suffix_len < 0 ||
      d->prefix_len > std::numeric_limits<int32_t>::max() ||
      d->suffix_len > std::numeric_limits<int32_t>::max() || d->head_dim < 1)
    return ATTN_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(d->scale)) return ATTN_ERR_VALUE;
  return ATTN_OK;
}

void bifurcated_descs(const attn_bifurcated_desc_t *d, attn_desc_t *prefix, attn_desc_t *suffix) {
  // Prefix: one "sequence" whose query tokens are the S samples (Q [S][Hq][D]
  // is Q [1][S][Hq][D]); every sample sees the whole prefix, so not causal.
  *prefix = attn_desc_t{};
  prefix->batch = d->num_samples > 0 ? 1 : 0;
  prefix->q_len = d->num_samples > 0 ? d->num_samples : 1;
  prefix->num_q_heads = d->num_q_heads;
  prefix->num_kv_heads = d->num_kv_heads;
  prefix->head_dim = d->head_dim;
  prefix->causal = 0;
  prefix->max_kv_len = d->prefix_len;
  prefix->kv_lens = nullptr;
  prefix->scale = d->scale;
  prefix->chunk_len = 0;
  prefix->dtype = d->dtype;
  // Suffix: an ordinary decode of one token per sample over its own KV.
  *suffix = *prefix;
  suffix->batch = d->num_samples;
  suffix->q_len = 1;
  suffix->max_kv_len = d->suffix_len;
}

}  // namespace attn
