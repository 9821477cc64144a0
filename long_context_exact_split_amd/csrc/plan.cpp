// Host-side validation and KV partitioning (no HIP calls).
//
// The partitioner turns one decode call into workgroups.  Tree Attention
// computes one local energy per device and Star Attention one block per host;
// on one GPU the unit of parallel work is the workgroup.  By default the
// balanced layout of work_map.h is used: one workgroup per CU, each streaming
// an equal share of all (sequence, KV head, row block) segments' tokens, with
// the lengths read on the device, so ragged batches stay balanced.  A forced
// chunk_len gives fixed chunks of C tokens instead.
#include "plan.h"

#include <cmath>
#include <cstring>
#include <limits>

namespace attn {
namespace {

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// The element type as the integer a C caller stored.  A C enum object may
// hold any int, but loading a value outside the enumerators through the C++
// enum type is undefined, so the field is read as its bytes.
int dtype_code(const attn_dtype_t &t) {
  int v;
  static_assert(sizeof(v) == sizeof(t), "attn_dtype_t is an int");
  std::memcpy(&v, &t, sizeof v);
  return v;
}

}  // namespace

int items_per_cu(int kernel, int64_t units, int cu_count) {
  // Short shares on the vector-ALU kernel: each workgroup's load pipeline
  // starts and drains once per piece, and two workgroups per CU overlap one
  // another's start-up (measured: 512-token segments, 9% faster).
  if (kernel == 0 && units < (int64_t)cu_count * kShortShare) return 2 * kItemsPerCu;
  return kItemsPerCu;
}

attn_status_t validate_desc(const attn_desc_t *d) {
  if (!d) return ATTN_ERR_NULL;
  const int dt = dtype_code(d->dtype);
  if (dt != ATTN_BF16 && dt != ATTN_F32) return ATTN_ERR_DTYPE;
  if (d->batch < 0 || d->q_len < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
      d->num_q_heads % d->num_kv_heads != 0 || d->max_kv_len < 0 || d->max_kv_len > kMaxKvLen ||
      d->head_dim < 1)
    return ATTN_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(d->scale)) return ATTN_ERR_VALUE;
  if (d->causal != 0 && d->causal != 1) return ATTN_ERR_VALUE;
  if (d->chunk_len < 0 || d->chunk_len % kChunkQuantum != 0) return ATTN_ERR_VALUE;
  const int64_t R = (int64_t)(d->num_q_heads / d->num_kv_heads) * d->q_len;
  if (R > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

KvPaging dense_paging(const attn_desc_t *d) {
  KvPaging pg{};
  pg.seq_stride = (int64_t)d->num_kv_heads * d->max_kv_len * d->head_dim;
  return pg;
}

attn_status_t validate_paged(const attn_desc_t *d, const attn_paged_kv_t *paged, KvPaging *pg) {
  *pg = dense_paging(d);
  if (!paged) return ATTN_OK;
  pg->seq_stride = 0;
  const int64_t P = paged->page_size;
  if (P < 1 || P > (int64_t(1) << kMaxPageShift) || (P & (P - 1)) != 0) return ATTN_ERR_VALUE;
  if (paged->pages_per_seq < 1 || (int64_t)paged->pages_per_seq * P < d->max_kv_len)
    return ATTN_ERR_VALUE;
  if (paged->num_pages < 0 || paged->page_stride < 0 || paged->head_stride < 0 ||
      paged->token_stride < 0)
    return ATTN_ERR_VALUE;
  const bool any_kv = d->batch > 0 && d->max_kv_len > 0;
  if (any_kv && (paged->num_pages < 1 || !paged->block_table)) {
    return paged->block_table ? ATTN_ERR_VALUE : ATTN_ERR_NULL;
  }
  // Every row starts on a 16-byte boundary.
  const int64_t q = d->dtype == ATTN_BF16 ? 8 : 4;
  if (paged->page_stride % q || paged->head_stride % q || paged->token_stride % q)
    return ATTN_ERR_ALIGN;
  constexpr int64_t kLimit = int64_t(1) << 48;
  if (paged->page_stride > 0 && paged->num_pages > kLimit / paged->page_stride)
    return ATTN_ERR_VALUE;
  if (paged->head_stride > kLimit / d->num_kv_heads || paged->token_stride > kLimit / P)
    return ATTN_ERR_VALUE;
  pg->block_table = any_kv ? paged->block_table : nullptr;
  pg->num_pages = paged->num_pages;
  pg->page_stride = paged->page_stride;
  pg->head_stride = paged->head_stride;
  pg->token_stride = paged->token_stride;
  pg->pages_per_seq = paged->pages_per_seq;
  int shift = 0;
  while ((int64_t(1) << shift) < P) ++shift;
  pg->page_shift = shift;
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
  // More than one block of 32 rows: the shared-tile MFMA kernel, whose waves
  // own 32 rows each and read every K/V tile once for all of them.
  p->kernel = (mfma_available && d->dtype == ATTN_BF16 && R > kMaxValuRows)
                  ? (R > kMfmaRows ? 2 : 1) : 0;
  if (p->kernel == 0) {
    p->rows_per_block = R <= 1 ? 1 : R <= 2 ? 2 : R <= 4 ? 4 : 8;
  } else if (p->kernel == 1) {
    p->rows_per_block = kMfmaRows;
  } else {
    const int waves = (R + kMfmaRows - 1) / kMfmaRows;
    p->rows_per_block = kMfmaRows * (waves <= 2 ? 2 : waves <= 4 ? 4 : 8);
    p->threads_per_item = p->rows_per_block * 2;  // one 64-lane wave per 32 rows
  }
  p->row_blocks = (R + p->rows_per_block - 1) / p->rows_per_block;
  const int64_t segs = (int64_t)d->batch * d->num_kv_heads * p->row_blocks;
  const int64_t L = d->max_kv_len;
  if (L > 0 && segs > kMaxUnits / L) return ATTN_ERR_UNSUPPORTED;
  if (d->chunk_len > 0) {
    p->balanced = 0;
    p->chunk_len = d->chunk_len;
    p->chunks_per_seq = (int32_t)(L > 0 ? (L + d->chunk_len - 1) / d->chunk_len : 0);
    p->work_items = segs * p->chunks_per_seq;
  } else {
    p->balanced = 1;
    p->chunks_per_seq = 0;
    // Upper bound (all sequences full); causal row blocks count the keys
    // they see.
    const WorkMap shape = work_map(d, *p);
    const int64_t units = (int64_t)d->batch * seq_units(shape, L);
    int64_t W = (int64_t)cu_count * items_per_cu(p->kernel, units, cu_count);
    if (W > 65535) W = 65535;
    const int64_t by_size = (units + kMinPiece - 1) / kMinPiece;
    if (W > by_size) W = by_size;
    p->work_items = units > 0 ? W : 0;
    const int64_t per = p->work_items > 0 ? (units + W - 1) / W : 0;
    if (per > std::numeric_limits<int32_t>::max()) return ATTN_ERR_UNSUPPORTED;
    p->chunk_len = (int32_t)per;
  }
  if (p->work_items > std::numeric_limits<int32_t>::max()) return ATTN_ERR_UNSUPPORTED;
  const WorkMap m = work_map(d, *p);
  p->record_slots = record_slots(m);
  p->workspace_bytes = partial_bytes(p->record_slots * p->rows_per_block, d->head_dim);
  return ATTN_OK;
}

WorkMap work_map(const attn_desc_t *d, const attn_plan_t &p) {
  WorkMap m{};
  m.kv_lens = d->kv_lens;
  m.L_max = d->max_kv_len;
  m.B = d->batch;
  m.Hkv = d->num_kv_heads;
  m.row_blocks = p.row_blocks;
  m.mode = p.balanced ? 1 : 0;
  m.chunk_len = p.balanced ? 0 : p.chunk_len;
  m.n_chunks = p.chunks_per_seq;
  m.n_wg = p.balanced ? (int32_t)p.work_items : 0;
  // Only the shared-tile kernel's row blocks (up to 256 rows, prefill-sized
  // query blocks) differ enough in visible keys to matter.
  m.causal_rows = (p.balanced && d->causal && p.row_blocks > 1 && p.kernel == 2) ? 1 : 0;
  m.q_len = d->q_len;
  m.G = d->num_q_heads / d->num_kv_heads;
  m.R = p.rows;
  m.rpb = p.rows_per_block;
  return m;
}

size_t partial_bytes(int64_t records, int head_dim) {
  if (records <= 0) return 0;
  const size_t ml = (size_t)round_up(records * (int64_t)sizeof(float), 256);
  const size_t o = (size_t)round_up(records * (int64_t)head_dim * (int64_t)sizeof(float), 256);
  return 2 * ml + o;
}

attn_status_t validate_bifurcated(const attn_bifurcated_desc_t *d) {
  if (!d) return ATTN_ERR_NULL;
  const int dt = dtype_code(d->dtype);
  if (dt != ATTN_BF16) return dt == ATTN_F32 ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_DTYPE;
  if (d->num_samples < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
      d->num_q_heads % d->num_kv_heads != 0 || d->prefix_len < 0 || d->suffix_len < 0 ||
      d->prefix_len > kMaxKvLen || d->suffix_len > kMaxKvLen || d->head_dim < 1)
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

namespace attn {

attn_status_t validate_anchor(const attn_anchor_desc_t *d) {
  if (!d) return ATTN_ERR_NULL;
  const int dt = dtype_code(d->dtype);
  if (dt != ATTN_BF16) return dt == ATTN_F32 ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_DTYPE;
  if (d->num_blocks < 0 || d->block_len < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
      d->num_q_heads % d->num_kv_heads != 0 || d->anchor_len < 0 || d->anchor_len > kMaxKvLen ||
      d->head_dim < 1)
    return ATTN_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(d->scale)) return ATTN_ERR_VALUE;
  if ((int64_t)(d->num_q_heads / d->num_kv_heads) * d->block_len > kMaxRows)
    return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

void anchor_descs(const attn_anchor_desc_t *d, attn_desc_t *anchor, attn_desc_t *local) {
  attn_desc_t c{};
  c.batch = d->num_blocks;
  c.q_len = d->block_len;
  c.num_q_heads = d->num_q_heads;
  c.num_kv_heads = d->num_kv_heads;
  c.head_dim = d->head_dim;
  c.kv_lens = nullptr;
  c.scale = d->scale;
  c.chunk_len = 0;
  c.dtype = d->dtype;
  *anchor = c;
  anchor->causal = 0;               // every anchor key precedes the block
  anchor->max_kv_len = d->anchor_len;
  *local = c;
  local->causal = 1;                // query i sees the block's keys t <= i
  local->max_kv_len = d->block_len;
}

}  // namespace attn

namespace attn {

constexpr bool kMfmaPlans = true;  // dense query blocks go to the matrix-core kernels

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

attn_status_t check_inputs(const attn_desc_t *d, const void *q, const void *k, const void *v,
                           bool need_v) {
  attn_status_t st = validate_desc(d);
  if (st != ATTN_OK) return st;
  // An empty call may pass null tensors (torch gives empty tensors a null base).
  const bool any_q = d->batch > 0, any_kv = any_q && d->max_kv_len > 0;
  if ((any_q && !q) || (any_kv && (!k || (need_v && !v)))) return ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || (v && !aligned(v, 16))) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

attn_status_t check_outputs(const attn_desc_t *d, const float *o, const float *lse, bool need_o) {
  attn_status_t st = validate_desc(d);
  if (st != ATTN_OK) return st;
  if (!lse || (need_o && !o)) return ATTN_ERR_NULL;
  if (!aligned(lse, 4) || (o && !aligned(o, 4))) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

attn_status_t check_workspace(size_t need, const void *ws, size_t ws_bytes) {
  if (need > 0 && !ws) return ATTN_ERR_NULL;
  if (ws_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

attn_status_t set_workgroups(const attn_desc_t *d, int64_t W, attn_plan_t *p) {
  if (!p->balanced || W < 1 || W > 65535) return ATTN_ERR_VALUE;
  const WorkMap shape = work_map(d, *p);
  const int64_t units = (int64_t)d->batch * seq_units(shape, d->max_kv_len);
  const int64_t per = (units + W - 1) / W;
  if (per > std::numeric_limits<int32_t>::max()) return ATTN_ERR_UNSUPPORTED;
  p->work_items = units > 0 ? W : 0;
  p->chunk_len = (int32_t)per;
  const WorkMap m = work_map(d, *p);
  p->record_slots = record_slots(m);
  p->workspace_bytes = partial_bytes(p->record_slots * p->rows_per_block, d->head_dim);
  return ATTN_OK;
}

// Workgroups of the one-launch shared-prefix kernel given to the prefix alone,
// in eighths of the launch: -1 = from the cost estimate below, 0 = every
// workgroup takes a share of both parts.
#ifndef ATTN_BIF_PREFIX_EIGHTHS
#define ATTN_BIF_PREFIX_EIGHTHS -1
#endif

// How many of W workgroups should run the prefix (the rest run the suffix),
// or 0 for a share of both in every workgroup.  The prefix is matrix-core
// work and the suffix a stream from HBM, so the two run side by side on
// different CUs; the split follows their times on the whole GPU: 4·D flops
// per (query row, prefix key) at the shared-tile kernel's rate, against the
// suffix bytes at the decode kernels' rate.  The kernels measured here run
// about 128 flops in the time they stream one byte (0.9 PFLOP/s against
// 7 TB/s).  Rounded to whole rounds of the eight XCDs; a part that would get
// less than one round, or more than all but one, leaves the shared form.
int64_t bifurcated_prefix_workgroups(const attn_bifurcated_desc_t *d, int64_t W) {
  if (ATTN_BIF_PREFIX_EIGHTHS == 0 || W < 16) return 0;
  if (ATTN_BIF_PREFIX_EIGHTHS > 0) {
    const int64_t wp = W * ATTN_BIF_PREFIX_EIGHTHS / 8;
    return wp - wp % 8;
  }
  constexpr double kFlopsPerByte = 128.0;
  const double esz = d->dtype == ATTN_BF16 ? 2.0 : 4.0;
  const double rows = (double)d->num_samples * d->num_q_heads;  // every (sample, query head)
  const double pre_flops = 4.0 * d->head_dim * rows * (double)d->prefix_len;
  const double suf_bytes =
      2.0 * esz * d->head_dim * (double)d->num_samples * d->num_kv_heads * (double)d->suffix_len;
  const double tp = pre_flops / kFlopsPerByte, ts = suf_bytes;
  if (!(tp > 0.0) || !(ts > 0.0)) return 0;
  int64_t wp = (int64_t)(tp / (tp + ts) * (double)W / 8.0 + 0.5) * 8;
  if (wp < 8 || wp > W - 8) return 0;
  return wp;
}

attn_status_t bifurcated_plans(const attn_bifurcated_desc_t *d, int cu, BifPlans *b) {
  bifurcated_descs(d, &b->pre, &b->suf);
  attn_status_t st;
  if ((st = make_plan(&b->pre, cu, kMfmaPlans, &b->pp)) != ATTN_OK) return st;
  if ((st = make_plan(&b->suf, cu, kMfmaPlans, &b->sp)) != ATTN_OK) return st;
  // One launch for both parts when the prefix takes the shared-tile kernel's
  // 256-row blocks and the suffix is a decode of a few rows per KV head
  // (planned for the vector-ALU kernel; in the one launch it runs on the
  // 32-row matrix-core code): one 8-wave workgroup per CU (the shared tiles
  // need one workgroup per CU anyway), the CUs split between the parts by
  // bifurcated_prefix_workgroups, or each workgroup with a share of both.
  b->fused = b->pp.work_items > 0 && b->sp.work_items > 0 && b->pp.kernel == 2 &&
             b->pp.rows_per_block == 8 * kMfmaRows && b->sp.kernel == 0 && b->pp.balanced &&
             b->sp.balanced;
  b->workgroups = 0;
  if (b->fused) {
    // Split form if the estimate asks for it, else (or if a part's shares
    // would not fit the work map's 32-bit token ranges on its fewer
    // workgroups) the shared form, else two launches with their own plans.
    const attn_plan_t pp0 = b->pp, sp0 = b->sp;
    auto recut = [&](int64_t wp, int64_t ws) {
      b->pp = pp0;
      b->sp = sp0;
      return set_workgroups(&b->pre, wp, &b->pp) == ATTN_OK &&
             set_workgroups(&b->suf, ws, &b->sp) == ATTN_OK;
    };
    const int64_t wp = bifurcated_prefix_workgroups(d, cu);
    if (!((wp > 0 && recut(wp, cu - wp)) || recut(cu, cu))) {
      b->pp = pp0;
      b->sp = sp0;
      b->fused = false;
    } else {
      b->workgroups = cu;
    }
  }
  b->pre_bytes = (size_t)round_up((int64_t)b->pp.workspace_bytes, 256);
  b->total = b->pre_bytes + b->sp.workspace_bytes;
  return ATTN_OK;
}

// Each workgroup's share then starts at a segment's first unit (its first
// piece starts at token 0), so no workgroup boundary falls inside a segment.
bool whole_segment_pieces(const WorkMap &m) {
  if (m.mode != 1 || m.n_wg <= 0) return false;
  const int64_t U = total_units(m);
  for (int64_t w = 0; w < m.n_wg; ++w) {
    PieceCursor c = first_piece(m, U, w);
    Piece p;
    if (next_piece(m, w, c, &p) && p.t0 != 0) return false;
  }
  return true;
}

attn_status_t anchor_plans(const attn_anchor_desc_t *d, int cu, bool allow_fusion,
                           AnchorPlans *a) {
  anchor_descs(d, &a->anc, &a->loc);
  attn_status_t st;
  if ((st = make_plan(&a->anc, cu, kMfmaPlans, &a->ap)) != ATTN_OK) return st;
  if ((st = make_plan(&a->loc, cu, kMfmaPlans, &a->lp)) != ATTN_OK) return st;
  a->anc_bytes = (size_t)round_up((int64_t)a->ap.workspace_bytes, 256);
  a->total = a->anc_bytes + a->lp.workspace_bytes;
  a->fuse = allow_fusion && a->ap.work_items > 0 && a->lp.work_items > 0 && a->ap.kernel == 2 &&
            a->lp.kernel == 2 && a->ap.rows_per_block == a->lp.rows_per_block &&
            whole_segment_pieces(work_map(&a->anc, a->ap)) &&
            whole_segment_pieces(work_map(&a->loc, a->lp));
  return ATTN_OK;
}

}  // namespace attn
