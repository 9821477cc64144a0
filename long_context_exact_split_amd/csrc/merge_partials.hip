// Merge of the partial records and normalisation (gfx950): for every output
// row, the (m, l, o) records its pieces left are combined with the
// associative rule m = max(m_a, m_b), l = l_a e^(m_a-m) + l_b e^(m_b-m), o
// likewise (Tree Attention article, an energy view of attention: max and
// logsumexp are associative; Star Attention's phase 2 aggregates the same
// statistics at its query host), then O = o / l and lse = (m + log2 l) ln 2.
// The records of a row are found in closed form from the work map
// (work_map.h), which the split kernels followed.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace attn {
namespace {

// Where a merge row's records are: P pieces of its own segment (record index
// prow + c*pstride) and S pieces of the shared call (srow + c*sstride).
struct RowRecords {
  int64_t prow, pstride, srow, sstride;
  int32_t P, S;
};

__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(x & 0xffffffff));
  const int hi = __builtin_amdgcn_readfirstlane((int)(x >> 32));
  return ((int64_t)hi << 32) | (uint32_t)lo;
}

// Run by a whole wave (the sums of sequence units are wave reductions);
// every lane gets the result, marked wave-uniform for the compiler.
// CAUSAL_ROWS = false: neither map has causal segment lengths (the launcher
// checked), and the copies below say so at compile time.
template <bool CAUSAL_ROWS>
__device__ __forceinline__ RowRecords row_records(const MergeArgs &a, int b, int kvh, int r) {
  WorkMap map = a.map, smap = a.smap;
  if constexpr (!CAUSAL_ROWS) {
    map.causal_rows = 0;
    smap.causal_rows = 0;
  }
  const int lane = threadIdx.x & (kWave - 1);
  int64_t tot = 0, pre = 0;
  if (map.mode != 0) {
    for (int bb = lane; bb < map.B; bb += kWave) {
      const int64_t u = seq_units(map, seq_len(map, bb));
      tot += u;
      pre += bb < b ? u : 0;
    }
    tot = wave_sum_i64(tot);
    pre = wave_sum_i64(pre);
  }
  RowRecords rr{};
  const int RBp = a.part.rows;
  const int64_t sigma = ((int64_t)b * map.Hkv + kvh) * map.row_blocks + r / RBp;
  const SlotRange pr = segment_slots_at(map, tot, pre, b, sigma);
  rr.P = (int32_t)pr.count;
  rr.prow = pr.first * RBp + r % RBp;
  rr.pstride = pr.stride * RBp;
  if (a.has_shared) {
    const int RBs = a.shared.rows;
    const int sb = a.shared_same_rows ? b : 0;              // sequence in the shared call
    const int rs = a.shared_same_rows ? r : b * a.R + r;  // row in that sequence
    const int64_t ssig = ((int64_t)sb * smap.Hkv + kvh) * smap.row_blocks + rs / RBs;
    const SlotRange sr = segment_slots(smap, total_units(smap), sb, ssig);
    rr.S = (int32_t)sr.count;
    rr.srow = sr.first * RBs + rs % RBs;
    rr.sstride = sr.stride * RBs;
  }
  rr.prow = uniform_i64(rr.prow);
  rr.pstride = uniform_i64(rr.pstride);
  rr.srow = uniform_i64(rr.srow);
  rr.sstride = uniform_i64(rr.sstride);
  rr.P = __builtin_amdgcn_readfirstlane(rr.P);
  rr.S = __builtin_amdgcn_readfirstlane(rr.S);
  return rr;
}

// The merge rule on one lane's share of two records: (ma, la, oa) becomes
// (ma, la, oa) + (mb, lb, ob).  The identity (-inf, 0, 0) is guarded
// (rescale_factor is 0 for a -inf maximum).
template <int N>
__device__ __forceinline__ void combine(float &ma, float &la, float (&oa)[N], float mb, float lb,
                                        const float (&ob)[N]) {
  const float M = fmaxf(ma, mb);
  const float fa = rescale_factor(ma, M), fb = rescale_factor(mb, M);
  la = la * fa + lb * fb;
#pragma unroll
  for (int e = 0; e < N; ++e) oa[e] = oa[e] * fa + ob[e] * fb;
  ma = M;
}

// Rows with many records (a long cache cut into many pieces, or a shared
// prefix cut into pieces for all samples): one workgroup per output row.
// The row's records are combined by a tree of the associative merge rule
// (Tree Attention article, an energy view of attention), in a fixed order:
//   * record groups of LPR lanes (16 bytes of o per lane); group g takes
//     records g, g + NG, g + 2NG, ... and loads up to kBatch of them at once
//     (one memory round trip for up to NG * kBatch records);
//   * each group reduces its batch as a binary tree in registers, and folds
//     the batch into what earlier batches left (rows with more than
//     NG * kBatch records);
//   * the groups of a wave pair up across lanes (v_permlane swaps), then the
//     waves' results pair up through LDS.
// Every wave works out where the row's records are by itself, so no barrier
// comes before the first record load.
constexpr int kMergeThreads = 256;
constexpr int kMergeWaves = kMergeThreads / kWave;
#ifndef ATTN_MERGE_BATCH
#define ATTN_MERGE_BATCH 8
#endif
constexpr int kBatch = ATTN_MERGE_BATCH;  // records per group loaded together

template <int D, bool ENERGY, bool CAUSAL_ROWS>
__global__ __launch_bounds__(kMergeThreads) void merge_partials(MergeArgs a) {
  constexpr int LPR = D / 4;                 // lanes per record (float4 each)
  constexpr int NG = kMergeThreads / LPR;    // record groups
  constexpr int EO = ENERGY ? 1 : 4;         // o elements per lane
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int64_t row = blockIdx.x;
  const int r = (int)(row % a.R);
  const int group = (int)(row / a.R);
  const int b = group / a.map.Hkv;
  const int kvh = group - b * a.map.Hkv;

  const RowRecords rr = row_records<CAUSAL_ROWS>(a, b, kvh, r);
  const int n = rr.P + rr.S;
  const int cg = tid / LPR;   // record group
  const int dl = tid % LPR;   // float4 slot within the record
  float Mg = -INFINITY, lg = 0.0f, og[EO];
#pragma unroll
  for (int e = 0; e < EO; ++e) og[e] = 0.0f;
  for (int c0 = 0; c0 < n; c0 += NG * kBatch) {
    float mc[kBatch], lc[kBatch], oc[kBatch][EO];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int c = c0 + cg + k * NG;
      mc[k] = -INFINITY;
      lc[k] = 0.0f;
#pragma unroll
      for (int e = 0; e < EO; ++e) oc[k][e] = 0.0f;
      if (c < n) {
        const bool shared = c >= rr.P;
        const int64_t rec = shared ? rr.srow + (c - rr.P) * rr.sstride : rr.prow + c * rr.pstride;
        // Pointers chosen as values: a reference to either argument struct
        // would be read back from argument memory before every record.
        mc[k] = (shared ? a.shared.m : a.part.m)[rec];
        lc[k] = (shared ? a.shared.l : a.part.l)[rec];
        if constexpr (!ENERGY) {
          const float4 v = *reinterpret_cast<const float4 *>(
              (shared ? a.shared.o : a.part.o) + rec * D + dl * 4);
          oc[k][0] = v.x;
          oc[k][1] = v.y;
          oc[k][2] = v.z;
          oc[k][3] = v.w;
        }
      }
    }
    // Binary tree over the batch: (0,1) (2,3) ..., then (01,23) ..., in place.
#pragma unroll
    for (int step = 1; step < kBatch; step *= 2)
#pragma unroll
      for (int k = 0; k + step < kBatch; k += 2 * step)
        combine<EO>(mc[k], lc[k], oc[k], mc[k + step], lc[k + step], oc[k + step]);
    combine<EO>(Mg, lg, og, mc[0], lc[0], oc[0]);
  }
  // Groups of one wave: lanes 16 and 32 apart hold the same slot of o of
  // neighbouring groups (LPR is 16 or 32); both lanes of a pair get the
  // lower lane's record first, so both combine the same two in one order.
  static_assert(LPR == 16 || LPR == 32, "head_dim 64 or 128");
  auto pair = [&](auto off_c) {
    constexpr int OFF = decltype(off_c)::value;
    float ma, mb, la, lb, oa[EO], ob[EO];
    lane_pair<OFF>(Mg, ma, mb);
    lane_pair<OFF>(lg, la, lb);
#pragma unroll
    for (int e = 0; e < EO; ++e) lane_pair<OFF>(og[e], oa[e], ob[e]);
    combine<EO>(ma, la, oa, mb, lb, ob);
    Mg = ma;
    lg = la;
#pragma unroll
    for (int e = 0; e < EO; ++e) og[e] = oa[e];
  };
  if constexpr (LPR == 16) pair(std::integral_constant<int, 16>{});
  pair(std::integral_constant<int, 32>{});
  // Waves: (0,1) and (2,3), then the two pairs.
  __shared__ float sm[kMergeWaves], sl[kMergeWaves];
  __shared__ float4 so[ENERGY ? 1 : kMergeWaves][ENERGY ? 1 : LPR];
  if (lane < LPR) {
    if (lane == 0) {
      sm[wave] = Mg;
      sl[wave] = lg;
    }
    if constexpr (!ENERGY) so[wave][lane] = make_float4(og[0], og[1], og[2], og[3]);
  }
  __syncthreads();
  if (wave != 0 || lane >= LPR) return;
  float wm[kMergeWaves], wl[kMergeWaves], wo[kMergeWaves][EO];
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) {
    wm[w] = sm[w];
    wl[w] = sl[w];
    if constexpr (!ENERGY) {
      const float4 v = so[w][lane];
      wo[w][0] = v.x;
      wo[w][1] = v.y;
      wo[w][2] = v.z;
      wo[w][3] = v.w;
    } else {
      wo[w][0] = 0.0f;
    }
  }
#pragma unroll
  for (int step = 1; step < kMergeWaves; step *= 2)
#pragma unroll
    for (int w = 0; w + step < kMergeWaves; w += 2 * step)
      combine<EO>(wm[w], wl[w], wo[w], wm[w + step], wl[w + step], wo[w + step]);

  const int i = r / a.G;
  const int h = kvh * a.G + (r - i * a.G);
  const int64_t orow = ((int64_t)b * a.q_len + i) * a.Hq + h;
  const bool empty = wm[0] == -INFINITY || !(wl[0] > 0.0f);
  if (lane == 0) a.lse[orow] = empty ? -INFINITY : (wm[0] + log2f(wl[0])) * kLn2;
  if constexpr (!ENERGY) {
    const float inv = empty ? 0.0f : 1.0f / wl[0];
    float *dst = a.o + orow * D + lane * 4;  // O is only 4-byte aligned
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = wo[0][e] * inv;
  }
}

// Rows with up to 32 records (most calls: a handful of pieces per segment): a
// wave per output row, or per run of rows_per_wave consecutive rows when
// there are hundreds of thousands of them (a prefill's query rows), four
// waves per workgroup.  Rows of one row block have their records in the same
// slots, one record row apart, so a run works out where they are once per
// block.  A row's records are loaded in batches and combined by a fixed tree
// of the merge rule (deterministic); each lane holds D/64 of the row's
// outputs.
constexpr int kRowsPerMergeBlock = 4;
// Records of one row loaded together (batches of 4 or 16 measured slower).
#ifndef ATTN_MERGE_ROW_BATCH
#define ATTN_MERGE_ROW_BATCH 8
#endif
constexpr int kRowBatch = ATTN_MERGE_ROW_BATCH;

template <int D, bool ENERGY, bool CAUSAL_ROWS>
__global__ __launch_bounds__(kRowsPerMergeBlock * kWave) void merge_rows(MergeArgs a,
                                                                          int rows_per_wave) {
  constexpr int EPL = D / kWave;  // output elements per lane
  constexpr int NO = ENERGY ? 1 : EPL;  // o elements carried per lane (a dummy when ENERGY)
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t rows = (int64_t)a.map.B * a.map.Hkv * a.R;
  const int64_t row0 =
      ((int64_t)blockIdx.x * kRowsPerMergeBlock + threadIdx.x / kWave) * rows_per_wave;
  if (row0 >= rows) return;  // whole waves; no workgroup barrier follows
  const int64_t row1 = row0 + rows_per_wave < rows ? row0 + rows_per_wave : rows;
  RowRecords rr{};
  int key_group = -1, key_p = -1, key_s = -1;  // the row blocks rr was worked out for
  for (int64_t row = row0; row < row1; ++row) {
    const int r = (int)(row % a.R);
    const int group = (int)(row / a.R);
    const int b = group / a.map.Hkv;
    const int kvh = group - b * a.map.Hkv;
    const int kp = r / a.part.rows;
    const int ks = a.has_shared ? (a.shared_same_rows ? r : b * a.R + r) / a.shared.rows : 0;
    if (group == key_group && kp == key_p && ks == key_s) {
      rr.prow += 1;  // the next row of the same blocks: the next record row
      rr.srow += 1;
    } else {
      rr = row_records<CAUSAL_ROWS>(a, b, kvh, r);
      key_group = group;
      key_p = kp;
      key_s = ks;
    }
    const int n = rr.P + rr.S;
    // Up to kRowBatch records are loaded at once (one memory round trip for
    // a row of that many) and combined as a binary tree, (0,1) (2,3) ...,
    // then pairs of pairs; the batch then joins what earlier batches left.
    // Slots past the row's count hold the identity record (-inf, 0, 0).
    float M = -INFINITY, lsum = 0.0f, acc[NO];
#pragma unroll
    for (int e = 0; e < NO; ++e) acc[e] = 0.0f;
    for (int c0 = 0; c0 < n; c0 += kRowBatch) {
      float mc[kRowBatch], lc[kRowBatch], oc[kRowBatch][NO];
#pragma unroll
      for (int k = 0; k < kRowBatch; ++k) {
        const int c = c0 + k;
        mc[k] = -INFINITY;
        lc[k] = 0.0f;
#pragma unroll
        for (int e = 0; e < NO; ++e) oc[k][e] = 0.0f;
        if (c < n) {
          const bool sh = c >= rr.P;
          const int64_t rec = sh ? rr.srow + (c - rr.P) * rr.sstride : rr.prow + c * rr.pstride;
          mc[k] = (sh ? a.shared.m : a.part.m)[rec];  // pointers as values, as above
          lc[k] = (sh ? a.shared.l : a.part.l)[rec];
          if constexpr (!ENERGY) {
            const float *po = (sh ? a.shared.o : a.part.o) + rec * D + lane * EPL;
#pragma unroll
            for (int e = 0; e < EPL; ++e) oc[k][e] = po[e];
          }
        }
      }
#pragma unroll
      for (int step = 1; step < kRowBatch; step *= 2)
#pragma unroll
        for (int k = 0; k + step < kRowBatch; k += 2 * step)
          combine<NO>(mc[k], lc[k], oc[k], mc[k + step], lc[k + step], oc[k + step]);
      combine<NO>(M, lsum, acc, mc[0], lc[0], oc[0]);
    }
    const int i = r / a.G;
    const int h = kvh * a.G + (r - i * a.G);
    const int64_t orow = ((int64_t)b * a.q_len + i) * a.Hq + h;
    const bool empty = M == -INFINITY || !(lsum > 0.0f);
    if (lane == 0) a.lse[orow] = empty ? -INFINITY : (M + log2f(lsum)) * kLn2;
    if constexpr (!ENERGY) {
      const float inv = empty ? 0.0f : 1.0f / lsum;
      float *dst = a.o + orow * D + lane * EPL;  // O is only 4-byte aligned
#pragma unroll
      for (int e = 0; e < EPL; ++e) dst[e] = acc[e] * inv;
    }
  }
}

// Waves that keep the whole GPU busy (256 CUs x 32): row runs get longer only
// beyond that many rows.
constexpr int64_t kMergeWavesWanted = 8192;
constexpr int kMaxRowsPerWave = 16;

// Rows whose record count exceeds this use the workgroup-per-row merge (the
// shared-prefix batch's rows of 18 records: wave per row 2 us faster than a
// workgroup per row; the 1M decode's rows of 33: a workgroup per row).
#ifndef ATTN_MERGE_WIDE_RECORDS
#define ATTN_MERGE_WIDE_RECORDS 32
#endif
constexpr int64_t kMergeWideRecords = ATTN_MERGE_WIDE_RECORDS;

// Records per output row, roughly, of a work map: fixed chunks give
// n_chunks; the balanced layout gives about W / segments + 1.
int64_t records_per_row(const WorkMap &m) {
  const int64_t segs = (int64_t)m.B * m.Hkv * m.row_blocks;
  if (segs <= 0) return 0;
  if (m.mode == 0) return m.n_chunks;
  return (int64_t)m.n_wg / segs + 1;
}

template <int D, bool ENERGY, bool CAUSAL_ROWS>
void launch_merge_dc(const MergeArgs &a, int64_t rows, bool wide, hipStream_t stream) {
  if (wide) {
    hipLaunchKernelGGL((merge_partials<D, ENERGY, CAUSAL_ROWS>), dim3((unsigned)rows),
                       dim3(kMergeThreads), 0, stream, a);
  } else {
    int rpw = 1;
    while (rpw < kMaxRowsPerWave && rows / (2 * rpw) >= kMergeWavesWanted) rpw *= 2;
    const int64_t waves = (rows + rpw - 1) / rpw;
    const int64_t blocks = (waves + kRowsPerMergeBlock - 1) / kRowsPerMergeBlock;
    hipLaunchKernelGGL((merge_rows<D, ENERGY, CAUSAL_ROWS>), dim3((unsigned)blocks),
                       dim3(kRowsPerMergeBlock * kWave), 0, stream, a, rpw);
  }
}

template <int D, bool ENERGY>
void launch_merge_d(const MergeArgs &a, int64_t rows, bool wide, hipStream_t stream) {
  if (a.map.causal_rows || (a.has_shared && a.smap.causal_rows))
    launch_merge_dc<D, ENERGY, true>(a, rows, wide, stream);
  else
    launch_merge_dc<D, ENERGY, false>(a, rows, wide, stream);
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, int head_dim, hipStream_t stream) {
  const int64_t rows = (int64_t)a.map.B * a.map.Hkv * a.R;
  if (rows == 0) return hipSuccess;
  // Few records per row: a wave per row; many: a workgroup per row.
  const int64_t per_row = records_per_row(a.map) + (a.has_shared ? records_per_row(a.smap) : 0);
  const bool wide = per_row > kMergeWideRecords;
  const bool energy = a.o == nullptr;
  if (head_dim == 64) {
    if (energy) launch_merge_d<64, true>(a, rows, wide, stream);
    else launch_merge_d<64, false>(a, rows, wide, stream);
  } else {
    if (energy) launch_merge_d<128, true>(a, rows, wide, stream);
    else launch_merge_d<128, false>(a, rows, wide, stream);
  }
  return hipGetLastError();
}

}  // namespace attn
