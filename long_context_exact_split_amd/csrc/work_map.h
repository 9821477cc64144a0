// Mapping between workgroups, KV segments and partial records (host and
// device code; the kernels and the host-side tests run this same code).
//
// A segment is one (sequence b, KV head, row block): the L_b cached tokens of
// that KV head, read for one block of query rows.  Segments are numbered
//     sigma = (b * Hkv + kvh) * row_blocks + rb.
// Two ways of cutting the segments into work:
//
// * fixed chunks (mode 0): workgroup w = sigma * n_chunks + c covers tokens
//   [c*C, min((c+1)*C, L_b)) of segment sigma; record slot = w.
//
// * balanced (mode 1): the segments are laid end to end into U token units
//   (sequence by sequence, KV head by KV head, and within a KV head the row
//   blocks in layout order, see block_at), and workgroup w takes units
//   [floor(w*U/W), floor((w+1)*U/W)).  A segment is as long as the keys its
//   rows can see: L_b, or under a causal mask with several row blocks of the
//   shared-tile kernel the keys visible to the block's last row (block_keys),
//   so that a prefill's early row blocks, which see few keys, are not given
//   as much work as the late ones.  Every workgroup then streams the same
//   number of keys whatever the lengths are (they are read from kv_lens on
//   the device, so the host never needs them).  A workgroup's range may start
//   or end inside a segment and may cover several short segments; each piece
//   gives one record, stored at slot w + (the segment's index in layout
//   order).  The pieces form a monotone staircase in the (w, layout index)
//   grid, so distinct pieces never share a slot, and W + #segments slots
//   suffice.  (LeanAttention, among the related work on the Bifurcated
//   Attention page, balances decode work across the GPU in the same spirit.)
#pragma once

#include <stdint.h>

#if defined(__HIP__)  // compiled as HIP: usable from kernels and host code
#include <hip/hip_runtime.h>
#define ATTN_HD __host__ __device__ __forceinline__
#else
#define ATTN_HD inline
#endif

namespace attn {

struct WorkMap {
  const int32_t *kv_lens;  // device lengths (host copy in host-side use); null: all L_max
  int64_t L_max;
  int32_t B, Hkv, row_blocks;
  int32_t mode;       // 0: fixed chunks, 1: balanced
  int32_t chunk_len;  // mode 0
  int32_t n_chunks;   // mode 0
  int32_t n_wg;       // mode 1: number of workgroups W
  // Mode 1 under a causal mask with several row blocks of the shared-tile
  // kernel: row block rb holds query rows [rb*rpb, min(R, (rb+1)*rpb)); row r
  // is query token r / G, which sees keys t <= L_b - q_len + r / G.
  // causal_rows = 0: every segment is L_b long.  Kernels instantiated for
  // maps without it clear the field in their copy of the map, so that the
  // causal arithmetic folds away.
  int32_t causal_rows;
  int32_t q_len, G, R, rpb;
};

ATTN_HD int64_t seq_len(const WorkMap &m, int b) {
  int64_t L = m.kv_lens ? (int64_t)m.kv_lens[b] : m.L_max;
  return L < 0 ? 0 : (L > m.L_max ? m.L_max : L);
}

ATTN_HD int64_t segs_per_seq(const WorkMap &m) { return (int64_t)m.Hkv * m.row_blocks; }

// sum over i in [0, n) of floor((a*i + b) / c), for n, a, b >= 0 and c >= 1.
// The lattice points under the line y = (a*x + b) / c are counted column by
// column; after reducing a and b below c, the same points are counted row by
// row, which is the sum with a and c exchanged: the Euclidean algorithm on
// (a, c), so O(log c) steps.  The callers' arguments are row counts (a*n + b
// stays below 2^31, as R <= 2^16), so the divisions are 32-bit.
ATTN_HD int64_t floor_sum(int32_t n, int32_t c, int32_t a, int32_t b) {
  int64_t s = 0;
  while (n > 0) {
    if (a >= c) {
      s += (int64_t)(a / c) * ((int64_t)n * (n - 1) / 2);
      a %= c;
    }
    if (b >= c) {
      s += (int64_t)(b / c) * n;
      b %= c;
    }
    const int32_t top = a * n + b;  // the line's height at x = n
    if (top < c) break;
    n = top / c;
    b = top % c;
    const int32_t t = c;
    c = a;
    a = t;
  }
  return s;
}

// Keys row block rb sees in a sequence of L keys (its segment length).
ATTN_HD int64_t block_keys(const WorkMap &m, int64_t L, int64_t rb) {
  if (!m.causal_rows) return L;
  const int32_t end = ((int32_t)rb + 1) * m.rpb;
  const int32_t last = (end < m.R ? end : m.R) - 1;  // the block's last row (< 2^16)
  const int64_t v = L - m.q_len + last / m.G + 1;
  return v < 0 ? 0 : (v > L ? L : v);
}

// Keys of row blocks 0 .. n-1 together (0 <= n <= row_blocks), in closed form:
// a block r below the last one is full, so it sees max(0, c + floor((rpb*r +
// rpb - 1) / G)) keys with c = L - q_len + 1 (never more than L, as its last
// row's token is below q_len).  The terms grow with r; they are positive from
// r0 on.
ATTN_HD int64_t keys_before(const WorkMap &m, int64_t L, int64_t n) {
  if (!m.causal_rows) return L * n;
  int64_t last_block = 0;
  if (n == m.row_blocks && n > 0) {
    last_block = block_keys(m, L, n - 1);
    n -= 1;
  }
  const int64_t c = L - m.q_len + 1;
  int32_t r0 = 0;
  if (c < 1) {
    // Positive from rpb*r >= need; need <= G*q_len = R, so 32-bit.
    const int32_t need = (int32_t)((int64_t)m.G * (1 - c)) - (m.rpb - 1);
    r0 = need <= 0 ? 0 : (need + m.rpb - 1) / m.rpb;
  }
  const int32_t n32 = (int32_t)n;  // n <= row_blocks <= 2^16
  if (n32 <= r0) return last_block;
  if (m.rpb % m.G == 0) {
    // Whole tokens per block (tpb of them): block r sees c - 1 + tpb*(r+1)
    // keys, an arithmetic series.
    const int64_t tpb = m.rpb / m.G;
    return last_block + (int64_t)(n32 - r0) * (c - 1) +
           tpb * (((int64_t)n32 * (n32 + 1) - (int64_t)r0 * (r0 + 1)) / 2);
  }
  return last_block + (int64_t)(n32 - r0) * c + floor_sum(n32, m.G, m.rpb, m.rpb - 1) -
         floor_sum(r0, m.G, m.rpb, m.rpb - 1);
}

// Units of one KV head of a sequence of L keys, and of the whole sequence.
ATTN_HD int64_t head_units(const WorkMap &m, int64_t L) { return keys_before(m, L, m.row_blocks); }
ATTN_HD int64_t seq_units(const WorkMap &m, int64_t L) { return m.Hkv * head_units(m, L); }

// Order of the row blocks of one KV head in the layout.  Causal row blocks
// go in zigzag order 0, n-1, 1, n-2, ... (n = row_blocks): block j and block
// n-1-j together see about as many keys as any other such pair, so every
// stretch of the layout mixes short and long segments and workgroups end up
// with similar numbers of pieces, each of which costs a pipeline start and a
// record write.  Otherwise the natural order.
ATTN_HD int64_t block_at(const WorkMap &m, int64_t pos) {
  if (!m.causal_rows) return pos;
  const int64_t j = pos / 2;
  return (pos & 1) ? m.row_blocks - 1 - j : j;
}

ATTN_HD int64_t pos_of(const WorkMap &m, int64_t rb) {
  if (!m.causal_rows) return rb;
  const int64_t mirror = m.row_blocks - 1 - rb;
  return rb <= mirror ? 2 * rb : 2 * mirror + 1;
}

// Units of the layout positions before pos (0 <= pos <= row_blocks) of one
// KV head: for pos = 2j the pairs (i, n-1-i), i < j, which are the first j
// blocks and the last j; for pos = 2j+1 also block j.
ATTN_HD int64_t units_before(const WorkMap &m, int64_t L, int64_t pos) {
  if (!m.causal_rows) return L * pos;
  const int64_t j = pos / 2;
  const int64_t even = keys_before(m, L, j) + head_units(m, L) - keys_before(m, L, m.row_blocks - j);
  return (pos & 1) ? even + block_keys(m, L, j) : even;
}

// The layout position whose segment holds unit rem of a KV head's units
// (0 <= rem < head_units): the last position starting at or before rem.
ATTN_HD int64_t position_of(const WorkMap &m, int64_t L, int64_t rem) {
  if (!m.causal_rows) return rem / L;
  int64_t lo = 0, hi = m.row_blocks - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (units_before(m, L, mid) <= rem) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Total token units U of the balanced layout.  Without per-sequence lengths
// every sequence holds L_max tokens: one product instead of a loop over the
// batch (a loop of 64-bit arithmetic per sequence costs microseconds on the
// device for batches of dozens of sequences).
ATTN_HD int64_t total_units(const WorkMap &m) {
  if (!m.kv_lens) return (int64_t)m.B * seq_units(m, m.L_max);
  int64_t u = 0;
  for (int b = 0; b < m.B; ++b) u += seq_units(m, seq_len(m, b));
  return u;
}

// Workgroups that take a share of the U units: the planned n_wg, or U when
// the cached tokens (read on the device) come to fewer units than that; the
// others idle.  Every share is then non-empty, so the pieces of a segment sit
// in consecutive workgroups and hence consecutive slots, which is what the
// merge's closed form (segment_slots) counts.  (With more workgroups than
// units some shares would be empty, and the merge would read slots no piece
// wrote.)
ATTN_HD int64_t active_wgs(const WorkMap &m, int64_t U) {
  return U < (int64_t)m.n_wg ? U : (int64_t)m.n_wg;
}

// First unit of workgroup w (balanced): floor(w * U / W) over the W active
// workgroups; wg_start(w) = U for w >= W (an idle workgroup).  Exact in
// 64-bit arithmetic while U * W < 2^63 (the planner enforces U < 2^46 units,
// W < 2^16).
ATTN_HD int64_t wg_start(const WorkMap &m, int64_t U, int64_t w) {
  const int64_t W = active_wgs(m, U);
  return w >= W ? U : (w * U) / W;
}

// The workgroup whose range holds unit x (0 <= x < U): the largest w with
// floor(w*U/W) <= x, i.e. w*U < (x+1)*W, i.e. w = ((x+1)*W - 1) / U.
ATTN_HD int64_t wg_of_unit(const WorkMap &m, int64_t U, int64_t x) {
  return ((x + 1) * active_wgs(m, U) - 1) / U;
}

// One piece of work: tokens [t0, t1) of segment sigma (numbered
// (b * Hkv + kvh) * row_blocks + rb), record slot `slot`.  Slots number the
// segments in layout order: slot = w + (b * Hkv + kvh) * row_blocks + the
// segment's layout position, which grows along the layout as w does, so
// distinct pieces never share a slot.
struct Piece {
  int64_t sigma;
  int64_t t0, t1;
  int64_t slot;
  int32_t b, kvh, rb;
};

// Iterator over the pieces of workgroup w in the balanced layout.
struct PieceCursor {
  int64_t x, xe;  // remaining units [x, xe)
  int64_t PB;     // first unit of sequence b
  int32_t b;
};

ATTN_HD PieceCursor first_piece(const WorkMap &m, int64_t U, int64_t w) {
  PieceCursor c;
  c.x = wg_start(m, U, w);
  c.xe = wg_start(m, U, w + 1);
  c.PB = 0;
  c.b = 0;
  return c;
}

// Fills *p with the next piece of workgroup w and advances; false when done.
ATTN_HD bool next_piece(const WorkMap &m, int64_t w, PieceCursor &c, Piece *p) {
  if (c.x >= c.xe) return false;
  int64_t L = seq_len(m, c.b);
  int64_t Tk = head_units(m, L);
  if (!m.kv_lens && c.PB + m.Hkv * Tk <= c.x) {
    // Equal sequences: jump straight to the one holding unit x.
    const int64_t per_seq = m.Hkv * Tk;  // > 0 here
    const int64_t skip = (c.x - c.PB) / per_seq;
    c.PB += skip * per_seq;
    c.b += (int32_t)skip;
  }
  while (c.PB + m.Hkv * Tk <= c.x) {  // skip whole sequences (empty ones included)
    c.PB += m.Hkv * Tk;
    ++c.b;
    L = seq_len(m, c.b);
    Tk = head_units(m, L);
  }
  const int64_t within = c.x - c.PB;
  const int64_t kvh = within / Tk;  // Tk > 0 here
  const int64_t rem = within - kvh * Tk;
  const int64_t pos = position_of(m, L, rem);
  const int64_t rb = block_at(m, pos);
  const int64_t P = c.PB + kvh * Tk + units_before(m, L, pos);
  const int64_t len = block_keys(m, L, rb);
  const int64_t end = P + len < c.xe ? P + len : c.xe;
  const int64_t group = (int64_t)c.b * m.Hkv + kvh;
  p->sigma = group * m.row_blocks + rb;
  p->t0 = c.x - P;
  p->t1 = end - P;
  p->slot = w + group * m.row_blocks + pos;
  p->b = c.b;
  p->kvh = (int32_t)kvh;
  p->rb = (int32_t)rb;
  c.x = end;
  return true;
}

// Record slots of segment sigma of sequence b: slots first, first + stride,
// ..., count of them.
struct SlotRange {
  int64_t first, stride, count;
};

// As segment_slots below, with PB = the units of the sequences before b (the
// sum of seq_units over them) and U already known.
ATTN_HD SlotRange segment_slots_at(const WorkMap &m, int64_t U, int64_t PB, int b, int64_t sigma) {
  SlotRange r{0, 1, 0};
  const int64_t L = seq_len(m, b);
  if (L == 0) return r;
  if (m.mode == 0) {
    r.first = sigma * m.n_chunks;
    r.count = (L + m.chunk_len - 1) / m.chunk_len;
    if (r.count > m.n_chunks) r.count = m.n_chunks;
    return r;
  }
  const int64_t s_in_b = sigma - (int64_t)b * segs_per_seq(m);
  const int64_t kvh = s_in_b / m.row_blocks, rb = s_in_b - kvh * m.row_blocks;
  const int64_t len = block_keys(m, L, rb);
  if (len == 0) return r;  // the block's rows see no key: no piece, no record
  const int64_t pos = pos_of(m, rb);
  const int64_t P = PB + kvh * head_units(m, L) + units_before(m, L, pos);
  const int64_t w0 = wg_of_unit(m, U, P), w1 = wg_of_unit(m, U, P + len - 1);
  r.first = w0 + (sigma - rb + pos);
  r.count = w1 - w0 + 1;
  return r;
}

ATTN_HD SlotRange segment_slots(const WorkMap &m, int64_t U, int b, int64_t sigma) {
  int64_t PB = 0;
  if (m.mode != 0) {
    if (!m.kv_lens) {
      PB = (int64_t)b * seq_units(m, m.L_max);
    } else {
      for (int bb = 0; bb < b; ++bb) PB += seq_units(m, seq_len(m, bb));
    }
  }
  return segment_slots_at(m, U, PB, b, sigma);
}

// Number of record slots a layout needs.
ATTN_HD int64_t record_slots(const WorkMap &m) {
  const int64_t segs = (int64_t)m.B * segs_per_seq(m);
  if (m.mode == 0) return segs * m.n_chunks;
  return (segs == 0 || m.n_wg == 0) ? 0 : (int64_t)m.n_wg + segs - 1;
}

}  // namespace attn
