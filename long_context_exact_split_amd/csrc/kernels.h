// Internal launch interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_decode.h"

namespace attn {

// Where the partial (m, l, o) records of one decode call live in the
// workspace: m and l are [groups][chunks][Rp] floats (m in log2 units), o is
// [groups][chunks][Rp][D] floats; groups = B * Hkv, Rp = row_blocks * RB.
struct PartialLayout {
  float *m;
  float *l;
  float *o;
  int32_t chunks;   // chunk slots per group
  int32_t rows;     // Rp
};

struct SplitArgs {
  const void *q;
  const void *k;
  const void *v;
  const int32_t *kv_lens;  // device, may be null
  PartialLayout part;
  int64_t L_max;
  int32_t B, q_len, Hq, Hkv, G, R, row_blocks;
  int32_t chunk_len, n_chunks;
  int32_t causal;
  float scale_log2;  // scale * log2(e)
};

// Merge of every record of a row, then normalisation.  Row r of group
// (b, kvh) merges the chunk records [0, ceil(L_b / chunk_len)) of `part` and,
// when shared.m is not null, all shared.chunks records of `shared` at group
// kvh, row b * R + r (records computed once for every batch entry, e.g. a
// shared prefix whose query rows are all samples' rows).
struct MergeArgs {
  PartialLayout part;
  PartialLayout shared;
  const int32_t *kv_lens;  // device, may be null
  int64_t L_max;
  int32_t B, q_len, Hq, Hkv, G, R;
  int32_t chunk_len;
  float *o;                // may be null (energy only)
  float *lse;
};

hipError_t launch_split_valu(const attn_plan_t &plan, const SplitArgs &a, attn_dtype_t dtype,
                             int head_dim, bool energy_only, hipStream_t stream);
hipError_t launch_split_mfma(const attn_plan_t &plan, const SplitArgs &a, int head_dim,
                             bool energy_only, hipStream_t stream);
hipError_t launch_merge(const MergeArgs &a, int head_dim, hipStream_t stream);

}  // namespace attn
