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
// * balanced (mode 1): the segments are laid end to end (offset of sigma =
//   sum of the lengths before it) into U token units, and workgroup w takes
//   units [floor(w*U/W), floor((w+1)*U/W)).  Every workgroup then streams the
//   same number of tokens whatever the lengths are (they are read from
//   kv_lens on the device, so the host never needs them).  A workgroup's range
//   may start or end inside a segment and may cover several short segments;
//   each (w, sigma) piece gives one record, stored at slot w + sigma.  The
//   pieces form a monotone staircase in the (w, sigma) grid, so distinct
//   pieces never share a slot, and W + #segments slots suffice.  (LeanAttention,
//   among the related work on the Bifurcated Attention page, balances decode
//   work across the GPU in the same spirit.)
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
};

ATTN_HD int64_t seq_len(const WorkMap &m, int b) {
  int64_t L = m.kv_lens ? (int64_t)m.kv_lens[b] : m.L_max;
  return L < 0 ? 0 : (L > m.L_max ? m.L_max : L);
}

ATTN_HD int64_t segs_per_seq(const WorkMap &m) { return (int64_t)m.Hkv * m.row_blocks; }

// Total token units U of the balanced layout.
ATTN_HD int64_t total_units(const WorkMap &m) {
  int64_t u = 0;
  for (int b = 0; b < m.B; ++b) u += seq_len(m, b);
  return u * segs_per_seq(m);
}

// First unit of workgroup w (balanced): floor(w * U / W); wg_start(W) = U.
// Exact in 64-bit arithmetic while U * W < 2^63 (the planner enforces
// U < 2^46 units, W < 2^16).
ATTN_HD int64_t wg_start(const WorkMap &m, int64_t U, int64_t w) {
  return (w * U) / (int64_t)m.n_wg;
}

// The workgroup whose range holds unit x (0 <= x < U): the largest w with
// floor(w*U/W) <= x, i.e. w*U < (x+1)*W, i.e. w = ((x+1)*W - 1) / U.
ATTN_HD int64_t wg_of_unit(const WorkMap &m, int64_t U, int64_t x) {
  return ((x + 1) * (int64_t)m.n_wg - 1) / U;
}

// One piece of work: tokens [t0, t1) of segment sigma, record slot `slot`.
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
  const int64_t S = segs_per_seq(m);
  int64_t L = seq_len(m, c.b);
  while (c.PB + L * S <= c.x) {  // skip whole sequences (empty ones included)
    c.PB += L * S;
    ++c.b;
    L = seq_len(m, c.b);
  }
  const int64_t within = c.x - c.PB;
  const int64_t s_in_b = within / L;  // L > 0 here
  const int64_t P = c.PB + s_in_b * L;
  const int64_t end = P + L < c.xe ? P + L : c.xe;
  p->sigma = (int64_t)c.b * S + s_in_b;
  p->t0 = c.x - P;
  p->t1 = end - P;
  p->slot = w + p->sigma;
  p->b = c.b;
  p->kvh = (int32_t)(s_in_b / m.row_blocks);
  p->rb = (int32_t)(s_in_b % m.row_blocks);
  c.x = end;
  return true;
}

// Record slots of segment sigma of sequence b: slots first, first + stride,
// ..., count of them.
struct SlotRange {
  int64_t first, stride, count;
};

// As segment_slots below, with PB = sum of seq_len over sequences before b
// (and U) already known.
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
  const int64_t S = segs_per_seq(m);
  const int64_t P = PB * S + (sigma - (int64_t)b * S) * L;
  const int64_t w0 = wg_of_unit(m, U, P), w1 = wg_of_unit(m, U, P + L - 1);
  r.first = w0 + sigma;
  r.count = w1 - w0 + 1;
  return r;
}

ATTN_HD SlotRange segment_slots(const WorkMap &m, int64_t U, int b, int64_t sigma) {
  int64_t PB = 0;
  if (m.mode != 0)
    for (int bb = 0; bb < b; ++bb) PB += seq_len(m, bb);
  return segment_slots_at(m, U, PB, b, sigma);
}

// Number of record slots a layout needs.
ATTN_HD int64_t record_slots(const WorkMap &m) {
  const int64_t segs = (int64_t)m.B * segs_per_seq(m);
  if (m.mode == 0) return segs * m.n_chunks;
  return (segs == 0 || m.n_wg == 0) ? 0 : (int64_t)m.n_wg + segs - 1;
}

}  // namespace attn
