// Split-KV decode on the vector ALUs (gfx950, wave64).
//
// Each workgroup takes its pieces of work from the work map (work_map.h): a
// piece is a token range of one (sequence b, KV head, row block) segment.  It
// streams the piece's K and V rows from HBM exactly once and serves every
// query row of the GQA group from them, producing the piece's softmax
// statistics m = max s, l = sum e^(s-m) and the unnormalised output
// o = sum e^(s-m) v ("attention acceleration" concept page, section 2.1,
// online softmax; the pieces stand in for the per-device local energies of
// the Tree Attention article and the per-host blocks of Star Attention's
// phase 2).  The merge kernels (merge_partials.hip) combine the records.
//
// Lane layout: a key row of D elements is read by LPK lanes with one 16-byte
// load each, so a wave load covers KPW = 64 / LPK consecutive keys (1 KiB of
// contiguous memory for bf16, D = 128).  Each lane keeps its slice of every
// query row of the block in registers; the slice dot products are combined
// across the LPK lanes with DPP row operations.  Every group of LPK lanes runs
// its own online softmax over the keys it reads (tile-level rescaling, taken
// only when the running max grows by more than 2^8), and the key slots and
// waves are merged once at the end of the piece.
//
// Logits are kept in log2 units (scale * log2 e folded into one fp32
// multiply after the fp32 dot product), so exponentials are v_exp_f32.

#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "kv_rows.h"

#ifdef ATTN_WG_STAMPS
#include "probe/wg_stamps.h"  // per-workgroup clocks: measurement builds only
#else
#define ATTN_WG_STAMP()
#endif

namespace attn {
namespace {

#ifndef ATTN_SPLIT_WAVES
#define ATTN_SPLIT_WAVES 4   // waves per workgroup
#endif
#ifndef ATTN_SPLIT_KT_SMALL
#define ATTN_SPLIT_KT_SMALL 4  // keys per lane group per tile, blocks of <= 4 rows
#endif
#ifndef ATTN_SPLIT_KT_LARGE
#define ATTN_SPLIT_KT_LARGE 4  // keys per lane group per tile, blocks of 8 rows
#endif
#ifndef ATTN_SPLIT_NT
#define ATTN_SPLIT_NT 1      // K/V loads marked non-temporal: read once, kept out of the caches
#endif

constexpr int kWaves = ATTN_SPLIT_WAVES;

// Calls f(integral_constant<int, OFF>) for OFF, 2*OFF, 4*OFF, ... < 64.
template <int OFF, typename F>
__device__ __forceinline__ void for_lane_offsets(F &&f) {
  if constexpr (OFF < kWave) {
    f(std::integral_constant<int, OFF>{});
    for_lane_offsets<2 * OFF>(f);
  }
}
constexpr int kThreads = kWaves * kWave;
constexpr float kLazyRescale = 8.0f;  // log2 units: rescale only past a 256x growth

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load16(const void *p) {
  const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
  const u32x4 v = ATTN_SPLIT_NT ? __builtin_nontemporal_load(q) : *q;
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename T, int D>
struct Geometry {
  static constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane per 16-byte load
  static constexpr int LPK = D / EPL;              // lanes per key row
  static constexpr int KPW = kWave / LPK;          // keys per wave load
};

template <typename T>
__device__ __forceinline__ void widen(const uint4 &w, float (&f)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
    f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
    f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
  } else {
    f[0] = __builtin_bit_cast(float, w.x); f[1] = __builtin_bit_cast(float, w.y);
    f[2] = __builtin_bit_cast(float, w.z); f[3] = __builtin_bit_cast(float, w.w);
  }
}

// Slice dot product: bf16 pairs on v_dot2_f32_bf16 (exact products, fp32
// accumulation), fp32 on FMAs.
template <typename T>
__device__ __forceinline__ float slice_dot(const uint4 &q, const uint4 &k) {
  if constexpr (sizeof(T) == 2) {
    float acc = dot2_bf16(q.x, k.x, 0.0f);
    acc = dot2_bf16(q.y, k.y, acc);
    acc = dot2_bf16(q.z, k.z, acc);
    return dot2_bf16(q.w, k.w, acc);
  } else {
    float acc = __builtin_bit_cast(float, q.x) * __builtin_bit_cast(float, k.x);
    acc = fmaf(__builtin_bit_cast(float, q.y), __builtin_bit_cast(float, k.y), acc);
    acc = fmaf(__builtin_bit_cast(float, q.z), __builtin_bit_cast(float, k.z), acc);
    return fmaf(__builtin_bit_cast(float, q.w), __builtin_bit_cast(float, k.w), acc);
  }
}

// Reduce-scatter of RB per-row partial dot products over the LPK lanes of one
// key row: afterwards the lane holds the full sum of one row only
// (scatter_row gives which), so the softmax steps that follow run once per
// (key, row) on RB-times fewer lanes than after an all-reduce.  The steps are
// the butterfly of group_sum (quad xor 1, quad xor 2, half-row mirror, row
// mirror, then lanes 16 apart), each step keeping half of the lane's rows and
// pulling the partner's partials for them.  The partners of the two mirror
// steps sit at the reflected quad position, so the rows a lane keeps are
// chosen from its quad position XOR 3 in odd quads; with that choice every
// lane's sum is bit-identical to what group_sum leaves in it for its row.
__device__ __forceinline__ int quad_pos(int kl) { return (kl & 3) ^ (((kl >> 2) & 1) ? 3 : 0); }

template <int LPK, int RB>
__device__ __forceinline__ int scatter_row(int kl) {
  const int pq = quad_pos(kl);
  int r = 0;
  if constexpr (RB >= 2) r += (pq & 1) * (RB / 2);
  if constexpr (RB >= 4) r += ((pq >> 1) & 1) * (RB / 4);
  if constexpr (RB >= 8) r += (LPK >= 16 ? (((kl >> 2) ^ (kl >> 3)) & 1) : ((kl >> 2) & 1));
  return r;
}

template <int LPK, int RB>
__device__ __forceinline__ float row_scatter_sum(const float (&x)[RB], int kl) {
  static_assert(RB == 1 || RB == 2 || RB == 4 || RB == 8, "rows per block");
  static_assert(LPK >= 8 && LPK >= RB, "lanes per key row");
  const int pq = quad_pos(kl);
  float v[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) v[r] = x[r];
  // Step 1 (quad xor 1).
  if constexpr (RB >= 2) {
    const bool up = pq & 1;
#pragma unroll
    for (int k = 0; k < RB / 2; ++k) {
      const float keep = up ? v[RB / 2 + k] : v[k];
      const float send = up ? v[k] : v[RB / 2 + k];
      v[k] = keep + dpp_f32<kDppQuadXor1>(send);
    }
  } else {
    v[0] += dpp_f32<kDppQuadXor1>(v[0]);
  }
  // Step 2 (quad xor 2).
  if constexpr (RB >= 4) {
    const bool up = (pq >> 1) & 1;
#pragma unroll
    for (int k = 0; k < RB / 4; ++k) {
      const float keep = up ? v[RB / 4 + k] : v[k];
      const float send = up ? v[k] : v[RB / 4 + k];
      v[k] = keep + dpp_f32<kDppQuadXor2>(send);
    }
  } else {
    v[0] += dpp_f32<kDppQuadXor2>(v[0]);
  }
  // Step 3 (half-row mirror).
  if constexpr (RB >= 8) {
    const bool up = LPK >= 16 ? (((kl >> 2) ^ (kl >> 3)) & 1) : ((kl >> 2) & 1);
    const float keep = up ? v[1] : v[0];
    const float send = up ? v[0] : v[1];
    v[0] = keep + dpp_f32<kDppRowHalfMirror>(send);
  } else {
    v[0] += dpp_f32<kDppRowHalfMirror>(v[0]);
  }
  // Steps 4 and 5: all-reduce over the rest of the key row.
  if constexpr (LPK >= 16) v[0] += dpp_f32<kDppRowMirror>(v[0]);
  float pa, pb;
  if constexpr (LPK >= 32) {
    lane_pair<16>(v[0], pa, pb);
    v[0] = pa + pb;
  }
  if constexpr (LPK >= 64) {
    lane_pair<32>(v[0], pa, pb);
    v[0] = pa + pb;
  }
  return v[0];
}

template <int D, int RB, bool ENERGY>
struct ValuSmem {
  float m[kWaves][RB], l[kWaves][RB];
  float o[ENERGY ? 1 : kWaves][ENERGY ? 1 : RB][ENERGY ? 1 : D];
};

// One piece: tokens [c0, c1) of KV head kvh of sequence b, for row block rb;
// writes the piece's record at `slot`.  MODE: what is produced (SplitMode);
// with kEnergyZeta each logit gains zeta . v_t, zeta being the row's
// auxiliary vector (Tree Attention article, an energy view of attention: the
// energy's gradient in zeta at 0 is the attention output).
template <typename T, int D, int RB, int KT, SplitMode MODE, bool PAGED>
__device__ __forceinline__ void valu_piece(const SplitArgs &a, int b, int kvh, int rb, int c0,
                                           int c1, int64_t slot,
                                           ValuSmem<D, RB, MODE != SplitMode::kFull> &sh) {
  constexpr bool ENERGY = MODE != SplitMode::kFull;
  constexpr bool ZETA = MODE == SplitMode::kEnergyZeta;
  constexpr bool LOADV = MODE != SplitMode::kEnergy;
  using Geo = Geometry<T, D>;
  constexpr int EPL = Geo::EPL, LPK = Geo::LPK, KPW = Geo::KPW;
  constexpr int TK = KPW * KT;  // keys per wave tile

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int kr = lane / LPK;  // key slot in a wave load
  const int kl = lane % LPK;  // slice of the key row
  const int Lb = (int)seq_len(a.map, b);

  // Visibility limit per row (keys t < lim[r]) and the query slices.
  int lim[RB];
  int hi = c0;
  uint4 q[RB], z[ZETA ? RB : 1];
  const T *Q = static_cast<const T *>(a.q);
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int rg = rb * RB + r;
    int n = c0;
    q[r] = make_uint4(0, 0, 0, 0);
    if constexpr (ZETA) z[r] = make_uint4(0, 0, 0, 0);
    if (rg < a.R) {
      const int i = rg / a.G;
      const int h = kvh * a.G + (rg - i * a.G);
      n = a.causal ? Lb - a.q_len + i + 1 : Lb;
      n = n < c0 ? c0 : (n > c1 ? c1 : n);
      const int64_t qoff = (((int64_t)b * a.q_len + i) * a.Hq + h) * D + kl * EPL;
      q[r] = *reinterpret_cast<const uint4 *>(Q + qoff);
      if constexpr (ZETA) z[r] = *reinterpret_cast<const uint4 *>(static_cast<const T *>(a.zeta) + qoff);
    }
    lim[r] = n;
    hi = max(hi, n);
  }

  // Softmax state.  Full decode: every lane keeps (m, l, o) for all RB rows
  // (the o slices differ per lane).  Energy: after the reduce-scatter a lane
  // owns one row, my_row, and keeps (m, l) for it alone.
  constexpr int NS_ROWS = ENERGY ? 1 : RB;
  float m[NS_ROWS], l[NS_ROWS], o[RB][ENERGY ? 1 : EPL];
#pragma unroll
  for (int r = 0; r < NS_ROWS; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.0f;
  }
  if constexpr (!ENERGY) {
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[r][e] = 0.0f;
  }
  const int my_row = ENERGY ? scatter_row<LPK, RB>(kl) : 0;
  int my_lim = lim[0];
#pragma unroll
  for (int r = 1; r < RB; ++r) my_lim = my_row == r ? lim[r] : my_lim;

  const KvRows<PAGED, D> rows(a, b, kvh);
  const T *kbase = static_cast<const T *>(a.k) + rows.origin + kl * EPL;
  const T *vbase = LOADV ? static_cast<const T *>(a.v) + rows.origin + kl * EPL : nullptr;
  const int n_tiles = (hi - c0 + TK - 1) / TK;

  // Token of key slot j of a wave tile, clamped so masked keys read a valid row.
  auto token = [&](int tile, int j) {
    const int t = c0 + tile * TK + j * KPW + kr;
    return t < hi ? t : hi - 1;
  };
  auto lookup_tile = [&](int tile, int32_t (&pg)[KT]) {
#pragma unroll
    for (int j = 0; j < KT; ++j) pg[j] = rows.lookup(token(tile, j));
  };
  auto load_tile = [&](int tile, const int32_t (&pg)[KT], uint4 (&kd)[KT],
                       uint4 (&vd)[LOADV ? KT : 1]) {
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const int64_t off = rows.offset(token(tile, j), pg[j]);
      kd[j] = load16(kbase + off);
      if constexpr (LOADV) vd[j] = load16(vbase + off);
    }
  };

  // Loads run ahead of the arithmetic (tiles past the end read the last
  // visible row again, an L2 hit).  With K and V: the next tile's loads are
  // issued before the arithmetic on this one.  K only: a ring of NSTG = 3
  // register stages, each refilled with the tile one round later as soon as
  // it has been consumed, so two tiles are in flight (the same bytes per wave
  // as with K and V); stage indices are compile-time in the unrolled round,
  // so no register copy has to wait for a load.  (The K+V loop keeps the
  // copy form: unrolled, the branch of the lazy rescale makes the compiler
  // wait for every load in flight at the join.)  Paged caches: block-table
  // loads are issued a tile ahead of the K/V loads that use them.
  constexpr int NSTG = 3;
  constexpr int RSTEP = NSTG * kWaves;  // tiles per round of one wave (K only)
  auto next_of = [&](int tile) { return tile + kWaves < n_tiles ? tile + kWaves : tile; };

  auto compute = [&](int tile, const uint4 (&kc)[KT], const uint4 (&vc)[LOADV ? KT : 1]) {
    if constexpr (ENERGY) {
      // One row per lane: reduce-scatter the slice dot products, then the
      // masked online softmax of that row.
      float s[KT];
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        float x[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          if constexpr (ZETA)
            x[r] = slice_dot<T>(q[r], kc[j]) * a.scale_log2 + slice_dot<T>(z[r], vc[j]) * kLog2e;
          else
            x[r] = slice_dot<T>(q[r], kc[j]);
        }
        s[j] = row_scatter_sum<LPK, RB>(x, kl);
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        const int t = c0 + tile * TK + j * KPW + kr;
        s[j] = t < my_lim ? (ZETA ? s[j] : s[j] * a.scale_log2) : -INFINITY;
        tmax = fmaxf(tmax, s[j]);
      }
      if (__any(tmax > m[0] + kLazyRescale)) {
        const float mn = fmaxf(m[0], tmax);
        l[0] *= rescale_factor(m[0], mn);
        m[0] = mn;
      }
      const float mref = m[0] == -INFINITY ? 0.0f : m[0];
#pragma unroll
      for (int j = 0; j < KT; ++j) l[0] += fast_exp2(s[j] - mref);
    } else {
      float s[KT][RB];
#pragma unroll
      for (int j = 0; j < KT; ++j)
#pragma unroll
        for (int r = 0; r < RB; ++r) s[j][r] = group_sum<LPK>(slice_dot<T>(q[r], kc[j]));

      float tmax[RB];
#pragma unroll
      for (int r = 0; r < RB; ++r) tmax[r] = -INFINITY;
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        const int t = c0 + tile * TK + j * KPW + kr;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          s[j][r] = t < lim[r] ? s[j][r] * a.scale_log2 : -INFINITY;
          tmax[r] = fmaxf(tmax[r], s[j][r]);
        }
      }
      bool need = false;
#pragma unroll
      for (int r = 0; r < RB; ++r) need |= tmax[r] > m[r] + kLazyRescale;
      if (__any(need)) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const float mn = fmaxf(m[r], tmax[r]);
          const float alpha = rescale_factor(m[r], mn);
          l[r] *= alpha;
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[r][e] *= alpha;
          m[r] = mn;
        }
      }
      float mref[RB];
#pragma unroll
      for (int r = 0; r < RB; ++r) mref[r] = m[r] == -INFINITY ? 0.0f : m[r];
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        float vf[EPL];
        widen<T>(vc[j], vf);
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const float p = fast_exp2(s[j][r] - mref[r]);
          l[r] += p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[r][e] = fmaf(p, vf[e], o[r][e]);
        }
      }
    }
  };

  if constexpr (LOADV) {
    uint4 kc[KT], vc[KT];
    int32_t pn[KT];
    int tile = wave;
    if (tile < n_tiles) {
      int32_t pc[KT];
      lookup_tile(tile, pc);
      load_tile(tile, pc, kc, vc);
      lookup_tile(next_of(tile), pn);
    }
    for (; tile < n_tiles; tile += kWaves) {
      int32_t pnn[KT];
      if constexpr (PAGED) lookup_tile(next_of(next_of(tile)), pnn);
      uint4 kn[KT], vn[KT];
      load_tile(next_of(tile), pn, kn, vn);
      compute(tile, kc, vc);
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        kc[j] = kn[j];
        vc[j] = vn[j];
        if constexpr (PAGED) pn[j] = pnn[j];
      }
    }
  } else {
    uint4 kb[NSTG][KT], vb[NSTG][1];
    int32_t pb[NSTG][KT];
    if (wave < n_tiles) {
#pragma unroll
      for (int st = 0; st < NSTG; ++st) {
        int32_t p0[KT];
        lookup_tile(wave + st * kWaves, p0);
        load_tile(wave + st * kWaves, p0, kb[st], vb[st]);
        if constexpr (PAGED) lookup_tile(wave + st * kWaves + RSTEP, pb[st]);
      }
    }
    for (int base = wave; base < n_tiles; base += RSTEP) {
#pragma unroll
      for (int st = 0; st < NSTG; ++st) {
        const int tile = base + st * kWaves;
        if (tile >= n_tiles) break;  // wave-uniform
        compute(tile, kb[st], vb[st]);
        load_tile(tile + RSTEP, pb[st], kb[st], vb[st]);
        if constexpr (PAGED) lookup_tile(tile + 2 * RSTEP, pb[st]);
      }
    }
  }

  // Merge the KPW key slots of the wave (lanes with equal kl, hence the same
  // rows): pairs of lanes l, l ^ off for off = LPK .. 32, exchanged without
  // LDS (lane_pair); both lanes of a pair merge the same two records.
  for_lane_offsets<LPK>([&](auto off_c) {
    constexpr int OFF = decltype(off_c)::value;
    {
#pragma unroll
      for (int r = 0; r < NS_ROWS; ++r) {
        float ma, mb, la, lb;
        lane_pair<OFF>(m[r], ma, mb);
        lane_pair<OFF>(l[r], la, lb);
        const float M = fmaxf(ma, mb);
        const float fa = rescale_factor(ma, M), fb = rescale_factor(mb, M);
        l[r] = la * fa + lb * fb;
        if constexpr (!ENERGY) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            float oa, ob;
            lane_pair<OFF>(o[r][e], oa, ob);
            o[r][e] = oa * fa + ob * fb;
          }
        }
        m[r] = M;
      }
    }
  });

  // Merge the waves through LDS and write the piece's record (the barrier
  // keeps the previous piece's readers of the buffers ahead of these writes).
  auto &sm = sh.m;
  auto &sl = sh.l;
  auto &so = sh.o;
  __syncthreads();
  if (kr == 0) {
    if constexpr (ENERGY) {
      if (kl < RB) {  // lanes 0 .. RB-1 of a key row own distinct rows
        sm[wave][my_row] = m[0];
        sl[wave][my_row] = l[0];
      }
    } else {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) so[wave][r][kl * EPL + e] = o[r][e];
        if (kl == 0) {
          sm[wave][r] = m[r];
          sl[wave][r] = l[r];
        }
      }
    }
  }
  __syncthreads();
  const int64_t rec0 = slot * RB;
  constexpr int kOut = ENERGY ? RB : RB * D;
  for (int idx = threadIdx.x; idx < kOut; idx += kThreads) {
    const int r = ENERGY ? idx : idx / D;
    const int d = ENERGY ? 0 : idx - r * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm[w][r]);
    float acc = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = rescale_factor(sm[w][r], M);
      if constexpr (!ENERGY) acc += so[w][r][d] * f;
      lsum += sl[w][r] * f;
    }
    if constexpr (!ENERGY) __builtin_nontemporal_store(acc, &a.part.o[(rec0 + r) * D + d]);
    if (d == 0) {
      __builtin_nontemporal_store(M, &a.part.m[rec0 + r]);
      __builtin_nontemporal_store(lsum, &a.part.l[rec0 + r]);
    }
  }
}

template <typename T, int D, int RB, int KT, SplitMode MODE, bool PAGED>
__global__ __launch_bounds__(kThreads) void split_kv_valu(SplitArgs a) {
  ATTN_WG_STAMP();
  __shared__ ValuSmem<D, RB, MODE != SplitMode::kFull> sh;
  WorkMap m = a.map;
  m.causal_rows = 0;  // never set for this kernel's maps (the launcher checks)
  if (m.mode == 0) {
    const int w = blockIdx.x;
    const int sigma = w / m.n_chunks, c = w - sigma * m.n_chunks;
    const int group = sigma / m.row_blocks, rb = sigma - group * m.row_blocks;
    const int b = group / m.Hkv, kvh = group - b * m.Hkv;
    const int L = (int)seq_len(m, b);
    const int c0 = c * m.chunk_len;
    if (c0 >= L) return;  // past the sequence: the merge reads ceil(L_b / C) records only
    valu_piece<T, D, RB, KT, MODE, PAGED>(a, b, kvh, rb, c0, min(c0 + m.chunk_len, L), w, sh);
  } else {
    const int64_t U = total_units(m);
    PieceCursor cur = first_piece(m, U, blockIdx.x);
    Piece p;
    while (next_piece(m, blockIdx.x, cur, &p))
      valu_piece<T, D, RB, KT, MODE, PAGED>(a, p.b, p.kvh, p.rb, (int)p.t0, (int)p.t1, p.slot, sh);
  }
}

template <typename T, int D, int RB, SplitMode MODE, bool PAGED>
hipError_t launch_t(const attn_plan_t &plan, const SplitArgs &a, hipStream_t stream) {
  constexpr int KT = RB <= 4 ? ATTN_SPLIT_KT_SMALL : ATTN_SPLIT_KT_LARGE;
  if (plan.work_items <= 0) return hipSuccess;
  if (a.map.causal_rows) return hipErrorInvalidValue;
  hipLaunchKernelGGL((split_kv_valu<T, D, RB, KT, MODE, PAGED>), dim3((unsigned)plan.work_items),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D, SplitMode MODE, bool PAGED>
hipError_t launch_rb(const attn_plan_t &plan, const SplitArgs &a, hipStream_t stream) {
  switch (plan.rows_per_block) {
    case 1: return launch_t<T, D, 1, MODE, PAGED>(plan, a, stream);
    case 2: return launch_t<T, D, 2, MODE, PAGED>(plan, a, stream);
    case 4: return launch_t<T, D, 4, MODE, PAGED>(plan, a, stream);
    case 8: return launch_t<T, D, 8, MODE, PAGED>(plan, a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D>
hipError_t launch_mode(const attn_plan_t &plan, const SplitArgs &a, SplitMode mode,
                       hipStream_t stream) {
  const bool paged = a.pg.block_table != nullptr;
  switch (mode) {
    case SplitMode::kFull:
      return paged ? launch_rb<T, D, SplitMode::kFull, true>(plan, a, stream)
                   : launch_rb<T, D, SplitMode::kFull, false>(plan, a, stream);
    case SplitMode::kEnergy:
      return paged ? launch_rb<T, D, SplitMode::kEnergy, true>(plan, a, stream)
                   : launch_rb<T, D, SplitMode::kEnergy, false>(plan, a, stream);
    case SplitMode::kEnergyZeta:  // dense caches only
      return paged ? hipErrorInvalidValue
                   : launch_rb<T, D, SplitMode::kEnergyZeta, false>(plan, a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_split_valu(const attn_plan_t &plan, const SplitArgs &a, attn_dtype_t dtype,
                             int head_dim, SplitMode mode, hipStream_t stream) {
  if (head_dim != 64 && head_dim != 128) return hipErrorInvalidValue;
  if (dtype == ATTN_BF16)
    return head_dim == 64 ? launch_mode<uint16_t, 64>(plan, a, mode, stream)
                          : launch_mode<uint16_t, 128>(plan, a, mode, stream);
  return head_dim == 64 ? launch_mode<float, 64>(plan, a, mode, stream)
                        : launch_mode<float, 128>(plan, a, mode, stream);
}

}  // namespace attn
