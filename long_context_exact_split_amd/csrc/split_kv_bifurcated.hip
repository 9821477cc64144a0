// One launch for both parts of a shared-prefix batch (Bifurcated Attention,
// TL;DR: decode attention splits into one contraction over the shared
// prefix and one over each sample's own decoded KV, with the same flops and
// far less memory traffic than attending each sample over its own copy).
//
// One workgroup of 8 waves per CU.  The prefix runs on the shared-tile
// matrix-core code, which serves the query rows of all samples from every
// K/V tile (the prefix is read once); the suffix segments run four at a time
// (two waves each).  The planner either splits the CUs between the two
// parts (the first workgroups take prefix pieces, the others suffix
// segments: matrix-core work on some CUs while the others stream from HBM),
// or gives every workgroup a share of both.  A suffix segment is one sample's
// own decoded KV of one KV head: a few hundred keys for the G query heads of
// the group.  It runs on the 32-row matrix-core code with only G rows valid:
// the matrix cores have the capacity to spare, a 512-token segment took the
// same ~13 us per CU there as on the vector-ALU decode code (both bound by
// the segment's stream), and the two parts' shared memory then overlays
// within one 8-wave workgroup.  In the shared form half of the workgroups of
// every XCD run their prefix piece first and the other half their suffix
// share first, so that there too some CUs are busy on the matrix cores while
// others keep HBM streaming.  Both parts write their (m, l, o) records as
// their own kernels do (work_map.h, one map each, with the workgroup count
// of its part), and the merge kernel combines them.
#include "mfma_piece.h"

#ifdef ATTN_WG_STAMPS
#define ATTN_WG_STAMPS_READBACK attn_probe_wg_stamps_bif
#include "probe/wg_stamps.h"  // per-workgroup clocks: measurement builds only
#else
#define ATTN_WG_STAMP()
#endif

namespace attn {
namespace {

constexpr int kBifWaves = 8;  // the shared-tile code's 256-row blocks: 8 waves of 32 rows
constexpr int kBifThreads = kBifWaves * kWave;

// The suffix runs as kSufGroups groups of waves, each on a segment of its
// own (a segment's pieces carry a latency chain of their own: query loads,
// the first tiles, the epilogue; several in flight overlap them).
#ifndef ATTN_BIF_SUF_GROUPS
#define ATTN_BIF_SUF_GROUPS 4  // 2: 0.5-1 us slower per call on the 64-sample batch
#endif
constexpr int kSufGroups = ATTN_BIF_SUF_GROUPS;
constexpr int kSufWaves = kBifWaves / kSufGroups;

template <int D>
union BifSmem {
  mfma::RowsSmem<D, kBifWaves, false> pre;
  mfma::MfmaSmem<D, false, kSufWaves> suf[kSufGroups];
};

template <int D>
__global__ __launch_bounds__(kBifThreads) void split_kv_bifurcated(SplitArgs pre, SplitArgs suf) {
  ATTN_WG_STAMP();
  __shared__ BifSmem<D> sh;
  const int w = blockIdx.x;
  WorkMap pm = pre.map, sm = suf.map;
  pm.causal_rows = 0;  // neither part is causal (the launcher checks)
  sm.causal_rows = 0;
  // wl: the workgroup's index in the part's own map.
  auto prefix = [&](int wl) __attribute__((always_inline)) {
    const int64_t U = total_units(pm);
    PieceCursor cur = first_piece(pm, U, wl);
    Piece p;
    while (next_piece(pm, wl, cur, &p))
      mfma::rows_piece<D, kBifWaves, false, false>(pre, p.b, p.kvh, p.rb, (int)p.t0, (int)p.t1,
                                                   p.slot, sh.pre);
  };
  auto suffix = [&](int wl) __attribute__((always_inline)) {
    const int64_t U = total_units(sm);
    PieceCursor cur = first_piece(sm, U, wl);
    const int grp = threadIdx.x / (kSufWaves * kWave);  // wave-uniform
    // Pieces kSufGroups at a time, one per group (every group walks the same
    // cursor and keeps the piece of its own index); a group left without one
    // runs an empty piece (same barriers, nothing written).  The group's
    // piece is copied under a wave-uniform branch, not indexed out of an
    // array (which would put the array in scratch memory).
    for (;;) {
      Piece mine, q;
      bool have = false;
      if (!next_piece(sm, wl, cur, &mine)) break;
      have = grp == 0;
#pragma unroll
      for (int i = 1; i < kSufGroups; ++i) {
        if (!next_piece(sm, wl, cur, &q)) break;
        if (i == grp) {
          mine = q;
          have = true;
        }
      }
      const int t0 = (int)mine.t0;
      mfma::mfma_piece<D, false, false, kSufWaves>(suf, mine.b, mine.kvh, mine.rb, t0,
                                                  have ? (int)mine.t1 : t0, mine.slot,
                                                  sh.suf[grp], grp * kSufWaves * kWave, have);
    }
  };
  // Split launches (the two maps' workgroup counts add up to the grid) give
  // each workgroup one part: the first pm.n_wg the prefix, the rest the
  // suffix.  Otherwise every workgroup takes a share of both.
  const bool split = pm.n_wg + sm.n_wg == (int)gridDim.x;
  const bool suffix_first = !split && ((w / 8) & 1);
  const int ws = split ? w - pm.n_wg : w;  // index in the suffix map
  if (suffix_first) suffix(ws);
  if (!split || w < pm.n_wg) prefix(w);
  if (!suffix_first && (!split || w >= pm.n_wg)) suffix(ws);
}

template <int D>
hipError_t launch_d(const SplitArgs &pre, const SplitArgs &suf, int64_t wgs, hipStream_t stream) {
  hipLaunchKernelGGL((split_kv_bifurcated<D>), dim3((unsigned)wgs), dim3(kBifThreads), 0, stream,
                     pre, suf);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bifurcated(const SplitArgs &pre, const SplitArgs &suf, int head_dim,
                             int suffix_rows_per_block, int64_t workgroups, hipStream_t stream) {
  if (workgroups <= 0) return hipSuccess;
  if (pre.map.causal_rows || suf.map.causal_rows || pre.map.mode != 1 || suf.map.mode != 1 ||
      !((pre.map.n_wg == workgroups && suf.map.n_wg == workgroups) ||
        (pre.map.n_wg > 0 && suf.map.n_wg > 0 && pre.map.n_wg + suf.map.n_wg == workgroups)) ||
      pre.part.rows != mfma::kRows * kBifWaves || suf.map.row_blocks != 1 ||
      suf.part.rows != suffix_rows_per_block || suf.R > suffix_rows_per_block ||
      suffix_rows_per_block > mfma::kRows)
    return hipErrorInvalidValue;
  if (head_dim == 64) return launch_d<64>(pre, suf, workgroups, stream);
  if (head_dim == 128) return launch_d<128>(pre, suf, workgroups, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
