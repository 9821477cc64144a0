// Merge of the partial records and normalisation (gfx950): for every output
// row, the (m, l, o) records its pieces left are combined with the
// associative rule m = max(m_a, m_b), l = l_a e^(m_a-m) + l_b e^(m_b-m), o
// likewise (Tree Attention article, an energy view of attention: max and
// logsumexp are associative; Star Attention's phase 2 aggregates the same
// statistics at its query host), then O = o / l and lse = (m + log2 l) ln 2.
// The records of a row are found in closed form from the work map
// (work_map.h), which the split kernels followed.
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

// Rows with many records (a long cache cut into many pieces): one workgroup
// per output row.  The row's records are read in parallel: 16 bytes of o per
// lane, kMergeThreads / (D/4) record groups, each combining its records in
// one pass with the rule itself (running max, earlier sums rescaled when it
// grows), so no separate pass over the records' maxima has to come first.
// The groups' results are then combined through LDS in a fixed order
// (deterministic).  Every wave works out where the row's records are by
// itself, so no barrier comes before the first record load.
constexpr int kMergeThreads = 256;

template <int D, bool ENERGY, bool CAUSAL_ROWS>
__global__ __launch_bounds__(kMergeThreads) void merge_partials(MergeArgs a) {
  constexpr int LPR = D / 4;                 // lanes per record (float4 each)
  constexpr int NG = kMergeThreads / LPR;    // record groups
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int r = (int)(row % a.R);
  const int group = (int)(row / a.R);
  const int b = group / a.map.Hkv;
  const int kvh = group - b * a.map.Hkv;

  const RowRecords rr = row_records<CAUSAL_ROWS>(a, b, kvh, r);
  const int n = rr.P + rr.S;
  const int cg = tid / LPR;   // record group
  const int dl = tid % LPR;   // float4 slot within the record
  float Mg = -INFINITY, lg = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4  // four records of a group in flight (unroll 2: 2-8% slower, 8: 18%)
  for (int c = cg; c < n; c += NG) {
    const bool shared = c >= rr.P;
    const int64_t rec = shared ? rr.srow + (c - rr.P) * rr.sstride : rr.prow + c * rr.pstride;
    // Pointers chosen as values: a reference to either argument struct would
    // be read back from argument memory before every record.
    const float mc = (shared ? a.shared.m : a.part.m)[rec];
    const float lc = (shared ? a.shared.l : a.part.l)[rec];
    const float Mn = fmaxf(Mg, mc);
    const float fa = rescale_factor(Mg, Mn), fb = rescale_factor(mc, Mn);
    lg = lg * fa + lc * fb;
    if constexpr (!ENERGY) {
      const float4 v =
          *reinterpret_cast<const float4 *>((shared ? a.shared.o : a.part.o) + rec * D + dl * 4);
      acc.x = acc.x * fa + v.x * fb;
      acc.y = acc.y * fa + v.y * fb;
      acc.z = acc.z * fa + v.z * fb;
      acc.w = acc.w * fa + v.w * fb;
    }
    Mg = Mn;
  }
  __shared__ float sm[NG], sl[NG];
  __shared__ float4 so[ENERGY ? 1 : NG][ENERGY ? 1 : LPR];
  if (dl == 0) {
    sm[cg] = Mg;
    sl[cg] = lg;
  }
  if constexpr (!ENERGY) so[cg][dl] = acc;
  __syncthreads();

  const int i = r / a.G;
  const int h = kvh * a.G + (r - i * a.G);
  const int64_t orow = ((int64_t)b * a.q_len + i) * a.Hq + h;
  float M = sm[0];
#pragma unroll
  for (int g = 1; g < NG; ++g) M = fmaxf(M, sm[g]);
  float f[NG];
  float ltot = 0.0f;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    f[g] = rescale_factor(sm[g], M);
    ltot += sl[g] * f[g];
  }
  const bool empty = M == -INFINITY || !(ltot > 0.0f);
  if (tid == 0) a.lse[orow] = empty ? -INFINITY : (M + log2f(ltot)) * kLn2;
  if constexpr (!ENERGY) {
    if (tid < LPR) {
      float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float4 v = so[g][tid];
        t.x += v.x * f[g]; t.y += v.y * f[g]; t.z += v.z * f[g]; t.w += v.w * f[g];
      }
      const float inv = empty ? 0.0f : 1.0f / ltot;
      float *dst = a.o + orow * D + tid * 4;  // O is only 4-byte aligned
      dst[0] = t.x * inv; dst[1] = t.y * inv; dst[2] = t.z * inv; dst[3] = t.w * inv;
    }
  }
}

// Rows with few records (most calls: a handful of pieces per segment): a
// wave per output row, or per run of rows_per_wave consecutive rows when
// there are hundreds of thousands of them (a prefill's query rows), four
// waves per workgroup.  Rows of one row block have their records in the same
// slots, one record row apart, so a run works out where they are once per
// block.  A row's records are loaded together and combined one after another
// in index order with the merge rule (deterministic); each lane holds D/64 of
// the row's outputs.
constexpr int kRowsPerMergeBlock = 4;
constexpr int kRowBatch = 4;  // records of one row loaded together

template <int D, bool ENERGY, bool CAUSAL_ROWS>
__global__ __launch_bounds__(kRowsPerMergeBlock * kWave) void merge_rows(MergeArgs a,
                                                                          int rows_per_wave) {
  constexpr int EPL = D / kWave;  // output elements per lane
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
    // a row of that many), then combined in index order with the rule itself.
    float M = -INFINITY, lsum = 0.0f, acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    for (int c0 = 0; c0 < n; c0 += kRowBatch) {
      float mc[kRowBatch], lc[kRowBatch], oc[ENERGY ? 1 : kRowBatch][EPL];
#pragma unroll
      for (int k = 0; k < kRowBatch; ++k) {
        const int c = c0 + k;
        mc[k] = -INFINITY;
        lc[k] = 0.0f;
        if constexpr (!ENERGY)
#pragma unroll
          for (int e = 0; e < EPL; ++e) oc[k][e] = 0.0f;
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
      for (int k = 0; k < kRowBatch; ++k) {
        if (c0 + k >= n) break;
        const float Mn = fmaxf(M, mc[k]);
        const float fa = rescale_factor(M, Mn), fb = rescale_factor(mc[k], Mn);
        lsum = lsum * fa + lc[k] * fb;
        if constexpr (!ENERGY)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] = acc[e] * fa + oc[k][e] * fb;
        M = Mn;
      }
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

// Rows whose record count exceeds this use the workgroup-per-row merge.
#ifndef ATTN_MERGE_WIDE_RECORDS
#define ATTN_MERGE_WIDE_RECORDS 8
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
