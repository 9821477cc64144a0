// Device code of the matrix-core split-KV kernels (included by the kernels
// that run it: split_kv_mfma.hip, and the one-launch shared-prefix kernel).
// See split_kv_mfma.hip for the design.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "kv_rows.h"

namespace attn {
namespace mfma {
namespace {


#ifndef ATTN_MFMA_KPAD
#define ATTN_MFMA_KPAD 8    // K tile row padding in LDS (bf16 elements, multiple of 8)
#endif
#ifndef ATTN_MFMA_VPAD
#define ATTN_MFMA_VPAD 32   // V tile row padding in LDS (bf16 elements, multiple of 8)
#endif

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRows = 32;   // query rows per work item
constexpr int kTile = 32;   // keys per tile
constexpr float kLazyRescale = 8.0f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef float f32x4e __attribute__((ext_vector_type(4)));
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

template <int D>
struct Tiles {
  static constexpr int LPK = D / 8;          // lanes per key row (16 bytes each)
  static constexpr int KPI = kWave / LPK;    // keys per load instruction
  static constexpr int NL = kTile / KPI;     // load instructions per tile and tensor
  static constexpr int KS = D / 16;          // MFMA k-steps of Q.K (8 dims per lane half)
  static constexpr int NT = D / 32;          // 32-dim output tiles of O^T
  static constexpr int KROW = D + ATTN_MFMA_KPAD;  // LDS row pitch of the K tile (bf16 elements)
  // LDS row pitch of the V tile (bf16 elements): consecutive rows 16 banks
  // apart, so the two 16-lane groups of a transpose-read pass use disjoint banks.
  static constexpr int VROW = D + ATTN_MFMA_VPAD;
};

template <int D, bool ENERGY, int WAVES = kWaves>
struct Smem {
  uint16_t k[WAVES][kTile * Tiles<D>::KROW];
  uint16_t v[WAVES][ENERGY ? 1 : kTile * Tiles<D>::VROW];
};

template <int D, bool ENERGY, int WAVES = kWaves>
struct SmemOut {
  float m[WAVES][kRows];
  float l[WAVES][kRows];
  float o[ENERGY ? 1 : WAVES][ENERGY ? 1 : kRows][ENERGY ? 1 : D + 4];
};

// Marks the Q fragments as produced here (after the loads that filled them
// are known to be complete), so that the compiler's wait-count tracking does
// not carry them into the tile loop as outstanding loads: otherwise it waits
// for every prefetched tile in flight before the first Q.K MFMA of a tile.
template <int KS>
__device__ __forceinline__ void settle(bf16x8_t (&qf)[KS]) {
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 t = __builtin_bit_cast(u32x4, qf[s]);
    uint32_t a0 = t.x, a1 = t.y, a2 = t.z, a3 = t.w;
    asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3));
    qf[s] = __builtin_bit_cast(bf16x8_t, u32x4{a0, a1, a2, a3});
  }
}

// max(x[l], x[l ^ 32]) in every lane, by gfx950's lane-half swap (no LDS).
__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  lane_pair<32>(x, a, b);
  return fmaxf(a, b);
}

// Query fragments and scale such that the scale is positive: a negative scale
// is moved into Q (negating bf16 is exact), and a zero scale makes every logit
// zero, as zero queries with scale 1 do.
template <int KS>
__device__ __forceinline__ float positive_scale(bf16x8_t (&qf)[KS], float scale_log2) {
  if (scale_log2 > 0.0f) return scale_log2;
  const uint32_t flip = scale_log2 < 0.0f ? 0x80008000u : 0u;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 t = __builtin_bit_cast(u32x4, qf[s]);
    if (scale_log2 < 0.0f) {
      t.x ^= flip; t.y ^= flip; t.z ^= flip; t.w ^= flip;
    } else {
      t = u32x4{0, 0, 0, 0};
    }
    qf[s] = __builtin_bit_cast(bf16x8_t, t);
  }
  return scale_log2 < 0.0f ? -scale_log2 : 1.0f;
}

typedef __attribute__((ext_vector_type(2))) float f32x2_t;

// Two floats -> two fp16 (round to nearest even), packed.
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t));
}

// Scaling of the P.V product's fp16 operands: P * 2^kPvShift and
// V * 2^-kPvShift.  The lazy rescale keeps P <= 2^8, so P * 2^7 <= 2^15 stays
// below the fp16 maximum, and bf16 values of V in [2^-7, 8.3e6] map to
// normal fp16 values exactly.  The row sums are accumulated from the scaled
// P too and multiplied by 2^-7 (exact) before they leave the kernel.
constexpr float kPvShift = 7.0f;
constexpr float kPvDown = 0.0078125f;  // 2^-7

// Eight bf16 values of V (16 bytes) -> eight fp16 values of V * 2^-7.
__device__ __forceinline__ u32x4 v_to_f16(u32x4 w) {
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float lo = __builtin_bit_cast(float, w[e] << 16) * kPvDown;
    const float hi = __builtin_bit_cast(float, w[e] & 0xFFFF0000u) * kPvDown;
    r[e] = pack_f16(lo, hi);
  }
  return r;
}

// 16 bytes of a tile row in LDS.  Row pitches and column offsets are
// multiples of 8 elements, so the address is 16-byte aligned; stated here so
// that the store is one ds_write_b128 (the compiler otherwise splits it into
// two 8-byte ds_write2_b32).
__device__ __forceinline__ u32x4 *lds16(uint16_t *p) {
  return reinterpret_cast<u32x4 *>(__builtin_assume_aligned(p, 16));
}

// The three parts of one 32-key tile in one wave.
//
// qk_tile: S^T = K.Q^T (raw logits), K read from LDS (row pitch KROW).
// K fragments of a tile (A operand of S^T, one per k-step), read from LDS.
template <int D>
__device__ __forceinline__ void k_frags(const uint16_t *ks, bf16x8_t (&kf)[D / 16]) {
  using T = Tiles<D>;
  const int lane = threadIdx.x & (kWave - 1);
  const int h = lane >> 5;
  const int j = lane & 31;
#pragma unroll
  for (int s = 0; s < T::KS; ++s)
    kf[s] = __builtin_bit_cast(
        bf16x8_t, *reinterpret_cast<const u32x4 *>(ks + j * T::KROW + h * (D / 2) + 8 * s));
}

template <int D>
__device__ __forceinline__ f32x16_t qk_frags(const bf16x8_t (&kf)[D / 16],
                                             const bf16x8_t (&qf)[D / 16]) {
  f32x16_t sacc;
#pragma unroll
  for (int e = 0; e < 16; ++e) sacc[e] = 0.0f;
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], sacc, 0, 0, 0);
  return sacc;
}

template <int D>
__device__ __forceinline__ f32x16_t qk_tile(const uint16_t *ks, const bf16x8_t (&qf)[D / 16]) {
  bf16x8_t kf[D / 16];
  k_frags<D>(ks, kf);
  return qk_frags<D>(kf, qf);
}

// softmax_tile: masked online softmax of the lane's row over the tile
// (lane l: row l % 32, keys 8(e/4) + 4h + e%4); t0: token of the tile's
// first key; the row sees keys t < lim.  Updates m and lsum (the latter in
// units of 2^kPvShift), returns the factor alpha by which the unnormalised
// output must be rescaled before this tile's P.V is added, and (full decode)
// P^T * 2^kPvShift as fp16 fragments.  The
// scale is positive (positive_scale), so the max is taken on the raw logits,
// masked keys become -inf in place (only on tiles that reach past some row's
// limit), and the scale is fused into the exponent's argument.
//
// MASK: 0 = the tile is wholly visible to the wave's rows (no mask), 1 =
// mask in place, 2 = decide at run time.  With MASK < 2 the function has no
// branch, so the caller's scheduler can interleave it with matrix work.
template <bool ENERGY, int MASK = 2>
__device__ __forceinline__ float softmax_tile(f32x16_t sacc, int t0, int lim, float scale_log2,
                                              float &m, float &lsum, f16x8_t (&pf)[2]) {
  const int h = (threadIdx.x & (kWave - 1)) >> 5;
  if (MASK == 1 || (MASK == 2 && __any(t0 + kTile > lim))) {
    // Key t0 + 8(e/4) + 4h + e%4 is visible when its offset 8(e/4) + e%4
    // (a constant per entry) is below lim - t0 - 4h.
    const int vis = lim - t0 - 4 * h;
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = 8 * (e >> 2) + (e & 3) < vis ? sacc[e] : -INFINITY;
  }
  float tmax = fmaxf(fmaxf(sacc[0], sacc[1]), sacc[2]);
#pragma unroll
  for (int e = 3; e < 15; e += 2) tmax = fmaxf(fmaxf(tmax, sacc[e]), sacc[e + 1]);
  tmax = fmaxf(tmax, sacc[15]) * scale_log2;
  tmax = pair_max(tmax);  // lanes l and l + 32 hold halves of the row's keys
  float alpha = 1.0f;
  if constexpr (MASK == 2) {
    if (__any(tmax > m + kLazyRescale)) {
      const float mn = fmaxf(m, tmax);
      alpha = rescale_factor(m, mn);
      lsum *= alpha;
      m = mn;
    }
  } else {  // the same decision, as selects
    const bool need = __any(tmax > m + kLazyRescale);
    const float mn = need ? fmaxf(m, tmax) : m;
    alpha = need ? rescale_factor(m, mn) : 1.0f;
    lsum *= alpha;
    m = mn;
  }
  const float mref = (m == -INFINITY ? 0.0f : m) - kPvShift;
#pragma unroll
  for (int e = 0; e < 16; ++e) sacc[e] = fast_exp2(fmaf(sacc[e], scale_log2, -mref));
  // Row sum as a tree (a chain of 16 dependent adds would stall the wave).
  float ps[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ps[e] = sacc[2 * e] + sacc[2 * e + 1];
#pragma unroll
  for (int e = 0; e < 4; ++e) ps[e] += ps[e + 4];
  lsum += (ps[0] + ps[2]) + (ps[1] + ps[3]);
  if constexpr (!ENERGY) {
    // P^T fragments (B operand): k-step s holds accumulator entries 8s..8s+7.
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_f16(sacc[8 * s + 2 * e], sacc[8 * s + 2 * e + 1]);
      pf[s] = __builtin_bit_cast(f16x8_t, w);
    }
  }
  return alpha;
}

// pv_tile: O^T += V^T.P^T (fp16 operands, V * 2^-7 and P * 2^7).  V^T
// fragments (A operand) by transpose reads: in 16-lane group g, lane lg
// points at key k0 + lg/4, column n0 + 4(lg%4); it receives the four keys
// k0..k0+3 of column n0 + lg.
template <int D>
__device__ __forceinline__ void pv_tile(const uint16_t *vs, const f16x8_t (&pf)[2],
                                        f32x16_t (&oacc)[D / 32]) {
  using T = Tiles<D>;
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4, lg = lane & 15;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int n = 0; n < T::NT; ++n) {
      s16x4_t part[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int key = 16 * s + 8 * r + 4 * (g >> 1) + (lg >> 2);
        const int col = 32 * n + 16 * (g & 1) + 4 * (lg & 3);
        part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t *)(vs + key * T::VROW + col));
      }
      const f16x8_t vf = __builtin_shufflevector(__builtin_bit_cast(f16x4_t, part[0]),
                                               __builtin_bit_cast(f16x4_t, part[1]), 0, 1, 2, 3,
                                               4, 5, 6, 7);
      oacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[s], oacc[n], 0, 0, 0);
    }
  }
}

template <int D, bool ENERGY>
__device__ __forceinline__ void rescale_o(f32x16_t (&oacc)[ENERGY ? 1 : D / 32], float alpha) {
  if constexpr (!ENERGY) {
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[n][e] *= alpha;
  }
}

// A whole tile in order (S^T, softmax, O rescale, P.V); ks / vs: the tile in
// LDS (row pitches KROW / VROW).
template <int D, bool ENERGY>
__device__ __forceinline__ void tile_step(const uint16_t *ks, const uint16_t *vs,
                                          const bf16x8_t (&qf)[D / 16], int t0, int lim,
                                          float scale_log2, float &m, float &lsum,
                                          f32x16_t (&oacc)[ENERGY ? 1 : D / 32]) {
  f16x8_t pf[2];
  const float alpha = softmax_tile<ENERGY>(qk_tile<D>(ks, qf), t0, lim, scale_log2, m, lsum, pf);
  if (__any(alpha != 1.0f)) rescale_o<D, ENERGY>(oacc, alpha);
  if constexpr (!ENERGY) pv_tile<D>(vs, pf, oacc);
}

template <int D, bool ENERGY, int WAVES = kWaves>
union MfmaSmem {
  Smem<D, ENERGY, WAVES> t;
  SmemOut<D, ENERGY, WAVES> out;
};

// One piece: tokens [c0, c1) of KV head kvh of sequence b, for row block rb;
// writes the piece's record at `slot`: rows r < a.part.rows of the 32
// (a.part.rows = 32 here, or fewer when a call with fewer query rows per KV
// head keeps records of that many rows).  WAVES waves take the tiles in turn:
// threads tbase .. tbase + 64*WAVES - 1 of the workgroup, with shared memory
// `sh` of their own, so that two groups of waves can run two pieces side by
// side.  Every call passes the workgroup barriers the same number of times
// (three), so such groups stay in step; write = false runs a piece without
// writing its record (a group with no piece of its own takes an empty one).
template <int D, bool ENERGY, bool PAGED, int WAVES = kWaves>
__device__ __forceinline__ void mfma_piece(const SplitArgs &a, int b, int kvh, int rb, int c0,
                                           int c1, int64_t slot,
                                           MfmaSmem<D, ENERGY, WAVES> &sh, int tbase = 0,
                                           bool write = true) {
  using T = Tiles<D>;
  constexpr int LPK = T::LPK, KPI = T::KPI, NL = T::NL, KS = T::KS, NT = T::NT;

  const int tid = (int)threadIdx.x - tbase;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int h = lane >> 5;   // lane half
  const int j = lane & 31;   // query row owned by this lane (and key slot in A layouts)
  const int Lb = (int)seq_len(a.map, b);
  __syncthreads();  // the previous piece's epilogue is done with the shared buffers

  // This lane's query row and its visibility limit (keys t < lim).
  const int row = rb * kRows + j;
  const bool valid = row < a.R;
  int lim = c0;
  bf16x8_t qf[KS];
  if (valid) {
    const int i = row / a.G;
    const int head = kvh * a.G + (row - i * a.G);
    lim = a.causal ? Lb - a.q_len + i + 1 : Lb;
    lim = lim < c0 ? c0 : (lim > c1 ? c1 : lim);
    const uint16_t *q = static_cast<const uint16_t *>(a.q) +
                        (((int64_t)b * a.q_len + i) * a.Hq + head) * D + h * (D / 2);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4 *>(q + 8 * s));
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(bf16x8_t, u32x4{0, 0, 0, 0});
  }
  const float scale_log2 = positive_scale<KS>(qf, a.scale_log2);
  // Last visible key over the block's rows (row limits grow with the token index).
  int hi;
  {
    const int last = min(a.R, (rb + 1) * kRows) - 1;
    const int ilast = last / a.G;
    hi = a.causal ? Lb - a.q_len + ilast + 1 : Lb;
    hi = hi < c0 ? c0 : (hi > c1 ? c1 : hi);
  }

  float m = -INFINITY, lsum = 0.0f;
  f32x16_t oacc[ENERGY ? 1 : NT];
#pragma unroll
  for (int n = 0; n < (ENERGY ? 1 : NT); ++n)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[n][e] = 0.0f;

  const KvRows<PAGED, D> rows(a, b, kvh);
  const uint16_t *kg = static_cast<const uint16_t *>(a.k) + rows.origin + (lane % LPK) * 8;
  const uint16_t *vg =
      ENERGY ? nullptr : static_cast<const uint16_t *>(a.v) + rows.origin + (lane % LPK) * 8;
  uint16_t *ks = sh.t.k[wave];
  uint16_t *vs = sh.t.v[wave];
  const int n_tiles = (hi - c0 + kTile - 1) / kTile;

  // Token of load i of a tile, clamped so masked keys read a valid row.
  auto token = [&](int tile, int i) {
    const int t = c0 + tile * kTile + i * KPI + lane / LPK;
    return t < hi ? t : hi - 1;
  };
  auto lookup = [&](int tile, int32_t (&pg)[NL]) {
#pragma unroll
    for (int i = 0; i < NL; ++i) pg[i] = rows.lookup(token(tile, i));
  };
  u32x4 kr[NL], vr[ENERGY ? 1 : NL];
  auto load = [&](int tile, const int32_t (&pg)[NL]) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int64_t off = rows.offset(token(tile, i), pg[i]);
      kr[i] = load_nt(kg + off);  // streamed once: non-temporal (ordinary loads: 11% slower)
      if constexpr (!ENERGY) vr[i] = load_nt(vg + off);
    }
  };

  // Paged caches: block-table loads run one tile ahead of the K/V loads.
  int tile = wave;
  int32_t pn[NL];
  if (tile < n_tiles) {
    int32_t pc[NL];
    lookup(tile, pc);
    load(tile, pc);
    lookup(tile + WAVES, pn);
  }
  settle<KS>(qf);
  for (; tile < n_tiles; tile += WAVES) {
    // Stage this tile in LDS (the wave's previous LDS reads are complete:
    // LDS instructions of one wave execute in order).
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int key = i * KPI + lane / LPK;
      *lds16(ks + key * T::KROW + (lane % LPK) * 8) = kr[i];
      if constexpr (!ENERGY) *lds16(vs + key * T::VROW + (lane % LPK) * 8) = v_to_f16(vr[i]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int t0 = c0 + tile * kTile;
    int32_t pnn[NL];
    if constexpr (PAGED) lookup(tile + 2 * WAVES, pnn);
    if (tile + WAVES < n_tiles) load(tile + WAVES, pn);
    if constexpr (PAGED) {
#pragma unroll
      for (int i = 0; i < NL; ++i) pn[i] = pnn[i];
    }

    tile_step<D, ENERGY>(ks, vs, qf, t0, lim, scale_log2, m, lsum, oacc);
  }

  // Per-wave row statistics: lanes l and l + 32 hold the same m and halves of l.
  lsum = (lsum + __shfl_xor(lsum, 32)) * kPvDown;
  __syncthreads();  // every wave is done with its tile buffers
  if (h == 0) {
    sh.out.m[wave][j] = m;
    sh.out.l[wave][j] = lsum;
  }
  if constexpr (!ENERGY) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        sh.out.o[wave][j][32 * n + 8 * (e >> 2) + 4 * h + (e & 3)] = oacc[n][e];
  }
  __syncthreads();
  const int rows_out = a.part.rows;  // <= kRows
  const int64_t rec0 = slot * rows_out;
  const int n_out = ENERGY ? rows_out : rows_out * D;
  for (int idx = tid; write && idx < n_out; idx += WAVES * kWave) {
    const int r = ENERGY ? idx : idx / D;
    const int d = ENERGY ? 0 : idx - r * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sh.out.m[w][r]);
    float acc = 0.0f, ls = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float f = rescale_factor(sh.out.m[w][r], M);
      if constexpr (!ENERGY) acc += sh.out.o[w][r][d] * f;
      ls += sh.out.l[w][r] * f;
    }
    if constexpr (!ENERGY) __builtin_nontemporal_store(acc, &a.part.o[(rec0 + r) * D + d]);
    if (d == 0) {
      __builtin_nontemporal_store(M, &a.part.m[rec0 + r]);
      __builtin_nontemporal_store(ls, &a.part.l[rec0 + r]);
    }
  }
}

// ---------------------------------------------------------------------------
// Shared-tile variant for many query rows per KV head (R > 32): a workgroup of
// RW waves owns 32*RW rows, all waves walk the same keys, and each 32-key K/V
// tile is loaded into LDS once (cooperatively, six tile buffers, see the
// pipeline below) and used by every wave.  For a shared prefix this reads
// the prefix once for all samples instead of once per block of 32 rows.  No
// cross-wave merge: each wave writes the records of its own 32 rows (or, in
// the finalising form, merges them with another call's records and writes
// O and lse).
// ---------------------------------------------------------------------------
// LDS tile buffers of the shared-tile kernel, and how many iterations ahead
// of its first use a tile is stored into them (one barrier per two tiles).
constexpr int kRowsBufs = 6;
constexpr int kStoreAhead = 4;
#ifndef ATTN_ROWS_RING
#define ATTN_ROWS_RING 2        // register ring stages with eight waves (3: 1% slower)
#endif
#ifndef ATTN_ROWS_VALU_PER_MFMA
#define ATTN_ROWS_VALU_PER_MFMA 4  // softmax VALU instructions placed after each MFMA (5: ~1% slower)
#endif

template <int D, int RW, bool ENERGY>
union RowsSmem {
  struct {
    uint16_t k[kRowsBufs][kTile * Tiles<D>::KROW];
    uint16_t v[kRowsBufs][ENERGY ? 1 : kTile * Tiles<D>::VROW];
  } t;
  struct {
    float stage[RW][kRows * 32];  // epilogue: one 32 x 32 float slice per wave
    float coef[RW][5][kRows];     // finalising epilogue: per-row merge factors
  } ep;
};

// Finalising epilogue of a piece that is its segment's only piece, when
// the other call of the same rows (a.fin_map) also left one record per row:
// the two records are merged by the rule and in the order the merge kernel
// uses (this call's record first), and O and lse are written directly.
// m, lsum: the wave's row statistics (lane l: row l % 32); oacc: O^T.
template <int D, int RW>
__device__ __forceinline__ void finalize_rows(const SplitArgs &a, int b, int kvh, int rb, float m,
                                              float lsum, const f32x16_t (&oacc)[D / 32],
                                              RowsSmem<D, RW, false> &sh) {
  constexpr int NT = D / 32;
  constexpr int OP = 32;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int h = lane >> 5, j = lane & 31;
  const WorkMap &fm = a.fin_map;
  int64_t PB = 0;
  if (!fm.kv_lens) {
    PB = (int64_t)b * seq_units(fm, fm.L_max);
  } else {
    for (int bb = 0; bb < b; ++bb) PB += seq_units(fm, seq_len(fm, bb));
  }
  const int64_t sigma = ((int64_t)b * fm.Hkv + kvh) * fm.row_blocks + rb;
  const SlotRange sr = segment_slots_at(fm, total_units(fm), PB, b, sigma);
  const int64_t frec0 = sr.first * a.fin_part.rows + wave * kRows;  // the wave's first row
  const int row0 = rb * kRows * RW + wave * kRows;                  // ... in the call's rows
  float *coef = &sh.ep.coef[wave][0][0];
  if (h == 0) {
    const float ma = a.fin_part.m[frec0 + j], la = a.fin_part.l[frec0 + j];
    float M = -INFINITY, L = 0.0f;
    const float M1 = fmaxf(M, m);
    const float fa0 = rescale_factor(M, M1), fb0 = rescale_factor(m, M1);
    L = L * fa0 + lsum * fb0;
    M = M1;
    const float M2 = fmaxf(M, ma);
    const float fa1 = rescale_factor(M, M2), fb1 = rescale_factor(ma, M2);
    L = L * fa1 + la * fb1;
    M = M2;
    const bool empty = M == -INFINITY || !(L > 0.0f);
    coef[0 * kRows + j] = fa0;
    coef[1 * kRows + j] = fb0;
    coef[2 * kRows + j] = fa1;
    coef[3 * kRows + j] = fb1;
    coef[4 * kRows + j] = empty ? 0.0f : 1.0f / L;
    const int r = row0 + j;
    if (r < a.R) {
      const int i = r / a.G;
      const int hq = kvh * a.G + (r - i * a.G);
      a.fin_lse[((int64_t)b * a.q_len + i) * a.Hq + hq] = empty ? -INFINITY : (M + log2f(L)) * kLn2;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // O^T tiles to rows through the wave's LDS slice, as for the records;
  // lane l finishes rows 8q + l/8 (q = 0..3), four dims at a time.
  float *stage = sh.ep.stage[wave];
  const int swz_w = (j & 7) * 4;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      stage[j * OP + ((8 * (e >> 2) + 4 * h) ^ swz_w) + (e & 3)] = oacc[n][e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = q * kWave + lane;
      const int rr = idx >> 3, c4 = (idx & 7) * 4;
      const float4 v = *reinterpret_cast<const float4 *>(stage + rr * OP + (c4 ^ ((rr & 7) * 4)));
      const float4 va =
          *reinterpret_cast<const float4 *>(a.fin_part.o + (frec0 + rr) * D + 32 * n + c4);
      const int r = row0 + rr;
      if (r < a.R) {
        const int i = r / a.G;
        const int hq = kvh * a.G + (r - i * a.G);
        const int64_t orow = ((int64_t)b * a.q_len + i) * a.Hq + hq;
        const float fa0 = coef[0 * kRows + rr], fb0 = coef[1 * kRows + rr];
        const float fa1 = coef[2 * kRows + rr], fb1 = coef[3 * kRows + rr];
        const float inv = coef[4 * kRows + rr];
        float *dst = a.fin_o + orow * D + 32 * n + c4;  // O is only 4-byte aligned
        dst[0] = ((0.0f * fa0 + v.x * fb0) * fa1 + va.x * fb1) * inv;
        dst[1] = ((0.0f * fa0 + v.y * fb0) * fa1 + va.y * fb1) * inv;
        dst[2] = ((0.0f * fa0 + v.z * fb0) * fa1 + va.z * fb1) * inv;
        dst[3] = ((0.0f * fa0 + v.w * fb0) * fa1 + va.w * fb1) * inv;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

template <int D, int RW, bool ENERGY, bool PAGED, bool FIN = false>
__device__ __forceinline__ void rows_piece(const SplitArgs &a, int b, int kvh, int rb, int c0,
                                           int c1, int64_t slot, RowsSmem<D, RW, ENERGY> &sh) {
  using T = Tiles<D>;
  constexpr int KS = T::KS, NT = T::NT;
  constexpr int NTH = RW * kWave;
  constexpr int PIECES = kTile * D / 8;  // 16-byte pieces per tensor tile
  constexpr int PER = (PIECES + NTH - 1) / NTH;  // pieces per thread per tensor
  static_assert(PIECES % kWave == 0, "whole waves take part in the tile copy");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int h = lane >> 5;
  const int j = lane & 31;
  const int Lb = (int)seq_len(a.map, b);
  __syncthreads();  // the previous piece is done with the tile buffers

  const int row = rb * kRows * RW + wave * kRows + j;
  const bool valid = row < a.R;
  int lim = c0;
  bf16x8_t qf[KS];
  if (valid) {
    const int i = row / a.G;
    const int head = kvh * a.G + (row - i * a.G);
    lim = a.causal ? Lb - a.q_len + i + 1 : Lb;
    lim = lim < c0 ? c0 : (lim > c1 ? c1 : lim);
    const uint16_t *q = static_cast<const uint16_t *>(a.q) +
                        (((int64_t)b * a.q_len + i) * a.Hq + head) * D + h * (D / 2);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4 *>(q + 8 * s));
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(bf16x8_t, u32x4{0, 0, 0, 0});
  }
  const float scale_log2 = positive_scale<KS>(qf, a.scale_log2);
  int hi;
  {
    const int last = min(a.R, (rb + 1) * kRows * RW) - 1;
    const int ilast = last / a.G;
    hi = a.causal ? Lb - a.q_len + ilast + 1 : Lb;
    hi = hi < c0 ? c0 : (hi > c1 ? c1 : hi);
  }

  float m = -INFINITY, lsum = 0.0f;
  f32x16_t oacc[ENERGY ? 1 : NT];
#pragma unroll
  for (int n = 0; n < (ENERGY ? 1 : NT); ++n)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[n][e] = 0.0f;

  const KvRows<PAGED, D> rows(a, b, kvh);
  const uint16_t *kg = static_cast<const uint16_t *>(a.k) + rows.origin;
  const uint16_t *vg = ENERGY ? nullptr : static_cast<const uint16_t *>(a.v) + rows.origin;
  const int n_tiles = (hi - c0 + kTile - 1) / kTile;

  // Tiles in flight: a ring of NS register stages (tile t lives in stage
  // t % NS) feeding the LDS tile buffers.  Stage indices are compile-time
  // inside the unrolled inner loop, so the ring stays in registers.
  constexpr int NS = RW >= 8 ? ATTN_ROWS_RING : (RW >= 4 ? 2 : 1);
  constexpr int SA = kStoreAhead;
  u32x4 kr[NS][PER], vr[NS][ENERGY ? 1 : PER];
  // Token of this thread's copy piece i of a tile (clamped to a valid row).
  auto token = [&](int tile, int i) {
    const int p = threadIdx.x + i * NTH;
    const int t = c0 + tile * kTile + p / (D / 8);
    return t < hi ? t : hi - 1;
  };
  auto lookup = [&](int tile, int32_t (&pg)[PER]) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (PIECES % NTH != 0 && threadIdx.x + i * NTH >= PIECES) break;  // wave-uniform
      pg[i] = rows.lookup(token(tile, i));
    }
  };
  auto load = [&](int tile, const int32_t (&pg)[PER], u32x4 (&kd)[PER],
                  u32x4 (&vd)[ENERGY ? 1 : PER]) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = threadIdx.x + i * NTH;
      if (PIECES % NTH != 0 && p >= PIECES) break;  // wave-uniform
      const int64_t off = rows.offset(token(tile, i), pg[i]) + (p % (D / 8)) * 8;
      // Ordinary (temporal) loads: non-temporal ones measured 5-6% slower
      // here, both where row blocks share tiles and on a shared prefix.
      kd[i] = *reinterpret_cast<const u32x4 *>(kg + off);
      if constexpr (!ENERGY) vd[i] = *reinterpret_cast<const u32x4 *>(vg + off);
    }
  };
  auto store = [&](int buf, const u32x4 (&kd)[PER], const u32x4 (&vd)[ENERGY ? 1 : PER]) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = threadIdx.x + i * NTH;
      if (PIECES % NTH != 0 && p >= PIECES) break;  // wave-uniform
      const int key = p / (D / 8), col = (p % (D / 8)) * 8;
      *lds16(sh.t.k[buf] + key * T::KROW + col) = kd[i];
      if constexpr (!ENERGY) *lds16(sh.t.v[buf] + key * T::VROW + col) = v_to_f16(vd[i]);
    }
  };

  // Software pipeline over the tiles.  Iteration t issues, for this wave,
  //   P.V of tile t and S^T of tile t+2 (matrix cores) and
  //   the softmax of tile t+1 (vector ALUs),
  // three independent pieces of work that can overlap; the rescale of O that
  // the softmax of tile t+1 asks for is applied before the P.V of tile t+1.
  // LDS holds six tiles, tile x in buffer x % 6; iteration t stores tile t+4
  // from the register ring, and a workgroup barrier follows odd iterations
  // only.  Both hazards still cross a barrier: the K of tile t+2 read in
  // iteration t was stored in iteration t-2, and the buffer that iteration t
  // overwrites last held tile t-2, whose V was read in iteration t-2; a
  // barrier follows iteration t-2 or t-1, whichever is odd.  (A barrier per
  // iteration with four buffers ran 3% slower on long pieces.)  Tiles past
  // the last read the last visible row again, and the S^T of a tile past the
  // last is computed but never used.
  // Register ring: tile x lives in stage x % NS; paged caches: the
  // block-table loads of tile x are issued in iteration x - 3 - 2*NS, NS - 1
  // iterations before the K/V loads of x (iteration x - 4 - NS), so waiting
  // for them never waits for K/V loads still in the ring; their results live
  // in a ring of page-id stages (tile x in stage x % NS).
  auto kbuf = [&](int tile) { return sh.t.k[(unsigned)tile % kRowsBufs]; };
  auto vbuf = [&](int tile) { return sh.t.v[(unsigned)tile % kRowsBufs]; };
  int32_t pr[NS][PER];
  for (int s2 = 0; s2 < NS; ++s2)
    for (int i = 0; i < PER; ++i) pr[s2][i] = 0;
  f32x16_t sbuf[2];         // S^T of tile x in sbuf[x % 2]
  f16x8_t pf[2];            // P^T of tile t
  float pend = 1.0f;        // O rescale owed before the next P.V
  if (n_tiles > 0) {
    // Tiles 0..SA-1 into LDS, tiles SA..SA-1+NS into the register ring.
#pragma unroll
    for (int x = 0; x < SA; ++x) {
      int32_t p0[PER];
      lookup(x, p0);
      load(x, p0, kr[x % NS], vr[x % NS]);
      store(x % kRowsBufs, kr[x % NS], vr[x % NS]);
    }
    settle<KS>(qf);
#pragma unroll
    for (int x = SA; x < SA + NS; ++x) {
      int32_t p0[PER];
      lookup(x, p0);
      load(x, p0, kr[x % NS], vr[x % NS]);
    }
    if constexpr (PAGED) {
#pragma unroll
      for (int x = SA + NS; x <= SA - 2 + 2 * NS; ++x) lookup(x, pr[x % NS]);
    }
    __syncthreads();
    pend = softmax_tile<ENERGY>(qk_tile<D>(kbuf(0), qf), c0, lim, scale_log2, m, lsum, pf);
    sbuf[1] = qk_tile<D>(kbuf(1), qf);
  }
  // Tiles [0, full) are wholly visible to every row of this wave (no mask).
  int wave_lim = lim;
#pragma unroll
  for (int off = 1; off < kWave; off *= 2) wave_lim = min(wave_lim, __shfl_xor(wave_lim, off));
  const int full = (wave_lim - c0) / kTile;
  // The matrix and vector work of one iteration, interleaved: all eight K
  // fragment reads of S^T first (S^T is a chain of dependent MFMAs; with each
  // read issued just before its MFMA, every link waited out a whole LDS
  // latency), then each MFMA followed by a few VALU instructions of the
  // softmax, the V reads two at a time behind the MFMAs (the
  // sched_group_barrier sequence fixes this order within the iteration).
  // PAR = tile % 2: S^T of tile + 2 replaces that of tile (consumed by the
  // previous iteration's softmax), so the two S^T registers alternate roles
  // with no copy between iterations.
  auto body = [&](int tile, auto par, auto mask) {
    constexpr int PAR = decltype(par)::value;
    constexpr int MASK = decltype(mask)::value;
    __builtin_amdgcn_s_setprio(0);  // see the tile store below
    bf16x8_t kf[KS];
    k_frags<D>(kbuf(tile + 2), kf);
    if constexpr (!ENERGY) pv_tile<D>(vbuf(tile), pf, oacc);
    sbuf[PAR] = qk_frags<D>(kf, qf);
    pend = softmax_tile<ENERGY, MASK>(sbuf[1 - PAR], c0 + (tile + 1) * kTile, lim, scale_log2,
                                      m, lsum, pf);
    __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);  // the K reads
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // an S^T MFMA
      if constexpr (!ENERGY) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // V reads
      __builtin_amdgcn_sched_group_barrier(0x002, ATTN_ROWS_VALU_PER_MFMA, 0);  // softmax VALU
    }
#pragma unroll
    for (int i = 0; i < (ENERGY ? 0 : 2 * NT); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // a P.V MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, ATTN_ROWS_VALU_PER_MFMA, 0);  // softmax VALU
    }
  };
  // U iterations per unrolled round: a multiple of NS (ring stages), of the
  // buffer count and of 2, so stages and barrier parity are constants.
  constexpr int U = 6;
  static_assert(U % NS == 0 && U % kRowsBufs == 0 && U % 2 == 0,
                "ring stages, buffers and S^T registers cycle within U");
  for (int base = 0; base < n_tiles - 1; base += U) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int tile = base + k;
      if (tile >= n_tiles - 1) break;  // uniform across the workgroup
      if (__any(pend != 1.0f)) rescale_o<D, ENERGY>(oacc, pend);
      // tile % 2 == k % 2 (base is a multiple of U, which is even)
      if (tile + 1 < full) {
        if (k & 1) body(tile, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
        else body(tile, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
      } else {
        if (k & 1) body(tile, std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
        else body(tile, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
      }
      if constexpr (PAGED) lookup(tile + SA - 1 + 2 * NS, pr[(k + SA - 1) % NS]);
      const int st = (k + SA) % NS;  // stage of tile + SA (constant once unrolled)
      // The tile store and the next loads run at a raised wave priority, so
      // that the other wave of the SIMD, busy with its matrix and softmax
      // work, does not hold them back (anchor prefill 1-2% faster; the same
      // raise around the matrix and softmax work instead: no change).
      __builtin_amdgcn_s_setprio(1);
      store((unsigned)(tile + SA) % kRowsBufs, kr[st], vr[st]);
      load(tile + SA + NS, pr[st], kr[st], vr[st]);
      if (k & 1) __syncthreads();  // after odd tiles only
    }
  }
  __builtin_amdgcn_s_setprio(0);
  if (n_tiles > 0) {  // the last tile's P.V
    if (__any(pend != 1.0f)) rescale_o<D, ENERGY>(oacc, pend);
    if constexpr (!ENERGY) pv_tile<D>(vbuf(n_tiles - 1), pf, oacc);
  }
  __syncthreads();  // every wave is done with the tile buffers (the epilogue reuses them)

  lsum = (lsum + __shfl_xor(lsum, 32)) * kPvDown;
  if constexpr (FIN) {
    finalize_rows<D, RW>(a, b, kvh, rb, m, lsum, oacc, sh);
    return;
  }
  // Records are written with non-temporal stores (here and in the other
  // split kernels): the merge launch reads each once, and left in L2 as dirty
  // lines they lengthened the end-of-kernel write-back (shared-prefix call
  // 66.7 -> 65.4 us).
  const int64_t rec0 = slot * (kRows * RW) + wave * kRows;  // this wave's first row
  if (h == 0) {
    __builtin_nontemporal_store(m, &a.part.m[rec0 + j]);
    __builtin_nontemporal_store(lsum, &a.part.l[rec0 + j]);
  }
  if constexpr (!ENERGY) {
    // Each wave turns its O^T tiles into row-contiguous stores through its own
    // 32 x 32 float slice of the (now idle) tile buffers: lane l holds rows'
    // dims 8(e/4) + 4h + e%4 of tile n; after the exchange every lane writes
    // 16 contiguous bytes and each row's 32 dims form one 128-byte run.
    // Slice row pitch 32 floats; 4-float column groups are XOR-swizzled by
    // row (keeps float4 alignment, spreads the column writes over banks).
    constexpr int OP = 32;
    float *stage = sh.ep.stage[wave];
    const int swz_w = (j & 7) * 4;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        stage[j * OP + ((8 * (e >> 2) + 4 * h) ^ swz_w) + (e & 3)] = oacc[n][e];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int idx = q * kWave + lane;   // 256 float4 = 32 rows x 8
        const int rr = idx >> 3, c4 = (idx & 7) * 4;
        const float4 v = *reinterpret_cast<const float4 *>(stage + rr * OP + (c4 ^ ((rr & 7) * 4)));
        f32x4e *dst = reinterpret_cast<f32x4e *>(a.part.o + (rec0 + rr) * D + 32 * n + c4);
        __builtin_nontemporal_store(f32x4e{v.x, v.y, v.z, v.w}, dst);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

// Workgroups are dealt to the eight XCDs in turn (workgroup w runs on XCD
// w % 8), and each XCD has its own L2.  When a KV head's tiles are read by
// several row blocks (a prefill's query blocks), neighbouring pieces of the
// balanced layout share them, so the logical index is permuted to give each
// XCD one contiguous stretch of the layout (a bijection of [0, n)).  With
// one row block per KV head (a shared prefix) no piece shares tiles with
// another and the identity is kept: there the permutation measured 4%
// slower, against 3% faster on the anchor-block prefill.
__device__ __forceinline__ int xcd_local_index(int w, int n, bool shared_tiles) {
  if (!shared_tiles) return w;
  constexpr int kXcds = 8;
  const int x = w % kXcds, j = w / kXcds;
  const int q = n / kXcds, r = n % kXcds;
  return x * q + min(x, r) + j;
}

}  // namespace
}  // namespace mfma
}  // namespace attn
