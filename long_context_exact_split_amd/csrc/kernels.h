// Internal launch interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_decode.h"
#include "kv_paging.h"
#include "work_map.h"

namespace attn {

// Partial (m, l, o) records in the workspace: record (slot, r) of a work
// map holds rows r < rows of one segment piece; m and l are float[slots*rows]
// (m in log2 units), o is float[slots*rows][D].
struct PartialLayout {
  float *m;
  float *l;
  float *o;
  int32_t rows;  // rows per record slot (the rows of one row block)
};

struct SplitArgs {
  const void *q;
  const void *k;
  const void *v;
  const void *zeta;  // energy with an auxiliary vector per row (layout of q), or null
  KvPaging pg;
  WorkMap map;
  PartialLayout part;
  int32_t q_len, Hq, G, R;
  int32_t causal;
  float scale_log2;  // scale * log2(e)
  // Finalising split (shared-tile kernel, balanced layout only): every piece
  // of this call and of fin_map is a whole segment, fin_map has the same
  // sequences, rows and row blocks, and its one record per row (fin_part) is
  // merged with the piece's own before O and lse are written (fin_o,
  // fin_lse); no record is written and no merge launch follows.
  int32_t fin;
  WorkMap fin_map;
  PartialLayout fin_part;
  float *fin_o, *fin_lse;
};

// Merge of every record of a row, then normalisation.  Output row r of
// (b, kvh) merges the records of segment ((b*Hkv + kvh)*row_blocks + r/rows)
// and, when has_shared, the records a second split call left for it: with
// shared_same_rows, that call had the same sequences and rows (row r of
// sequence b); otherwise it was one sequence holding every sequence's rows,
// row b*R + r of KV head kvh (a shared prefix computed once for all samples).
struct MergeArgs {
  WorkMap map;
  PartialLayout part;
  int32_t has_shared;
  int32_t shared_same_rows;
  WorkMap smap;
  PartialLayout shared;
  int32_t q_len, Hq, G, R;
  float *o;  // may be null (energy only)
  float *lse;
};

// What a split launch produces: (m, l, o) records, (m, l) only, or (m, l) of
// the logits shifted by zeta . v (energy with zeta; vector-ALU kernel only).
enum class SplitMode { kFull, kEnergy, kEnergyZeta };

hipError_t launch_split_valu(const attn_plan_t &plan, const SplitArgs &a, attn_dtype_t dtype,
                             int head_dim, SplitMode mode, hipStream_t stream);
hipError_t launch_split_mfma(const attn_plan_t &plan, const SplitArgs &a, int head_dim,
                             bool energy_only, hipStream_t stream);
hipError_t launch_merge(const MergeArgs &a, int head_dim, hipStream_t stream);
// Both parts of a shared-prefix call in one launch of `workgroups` 8-wave
// workgroups: the prefix split (shared-tile code, 256-row blocks) and the
// suffix split (32-row matrix-core code, suffix_rows_per_block rows), each
// over its own balanced map: either both with n_wg == workgroups (every
// workgroup takes a share of both) or with the two n_wg adding up to
// workgroups (the first pre.map.n_wg take prefix pieces, the rest suffix
// segments); full mode, dense caches.  The merge is launched after it.
hipError_t launch_bifurcated(const SplitArgs &pre, const SplitArgs &suf, int head_dim,
                             int suffix_rows_per_block, int64_t workgroups, hipStream_t stream);

}  // namespace attn
