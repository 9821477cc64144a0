// Host-side views of the partition and of the argument checks, for tests
// (declared in attn_decode_testing.h).  Pure host code: it runs on the host
// the same partition arithmetic (work_map.h) the kernels run on the device,
// and the same checks the entry points run before any launch.  Linked into
// the test build of the library, never into the product library; the host
// sanitizer test compiles this file and plan.cpp alone.
#include <cstdint>

#include "attn_decode.h"
#include "attn_decode_testing.h"
#include "plan.h"

using namespace attn;

extern "C" {

int64_t attn_testing_pieces(const attn_desc_t *desc, const int32_t *host_lens, int32_t cu_count,
                            int64_t w, int64_t *out, int64_t max_pieces) {
  try {
    attn_plan_t p;
    attn_status_t st = make_plan(desc, cu_count, true, &p);
    if (st != ATTN_OK) return -(int64_t)st;
    if (w < 0 || w >= p.work_items || (!out && max_pieces > 0)) return -(int64_t)ATTN_ERR_VALUE;
    attn_desc_t d = *desc;
    d.kv_lens = host_lens;
    const WorkMap m = work_map(&d, p);
    int64_t n = 0;
    auto emit = [&](int64_t sigma, int64_t t0, int64_t t1, int64_t slot) {
      if (n < max_pieces) {
        out[4 * n] = sigma;
        out[4 * n + 1] = t0;
        out[4 * n + 2] = t1;
        out[4 * n + 3] = slot;
      }
      ++n;
    };
    if (m.mode == 0) {
      const int64_t sigma = w / m.n_chunks, c = w % m.n_chunks;
      const int b = (int)(sigma / segs_per_seq(m));
      const int64_t L = seq_len(m, b), c0 = c * m.chunk_len;
      if (c0 < L) emit(sigma, c0, c0 + m.chunk_len < L ? c0 + m.chunk_len : L, w);
    } else {
      const int64_t U = total_units(m);
      PieceCursor cur = first_piece(m, U, w);
      Piece pc;
      while (next_piece(m, w, cur, &pc)) emit(pc.sigma, pc.t0, pc.t1, pc.slot);
    }
    return n;
  } catch (...) {
    return -(int64_t)ATTN_ERR_HIP;
  }
}

attn_status_t attn_testing_segment_slots(const attn_desc_t *desc, const int32_t *host_lens,
                                         int32_t cu_count, int64_t segment, int64_t out[3]) {
  try {
    attn_plan_t p;
    attn_status_t st = make_plan(desc, cu_count, true, &p);
    if (st != ATTN_OK) return st;
    if (!out) return ATTN_ERR_NULL;
    attn_desc_t d = *desc;
    d.kv_lens = host_lens;
    const WorkMap m = work_map(&d, p);
    if (segment < 0 || segment >= (int64_t)m.B * segs_per_seq(m)) return ATTN_ERR_VALUE;
    const SlotRange r = segment_slots(m, total_units(m), (int)(segment / segs_per_seq(m)), segment);
    out[0] = r.first;
    out[1] = r.stride;
    out[2] = r.count;
    return ATTN_OK;
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

int32_t attn_testing_anchor_fuses(const attn_anchor_desc_t *desc, int32_t cu_count) {
  try {
    attn_status_t st = validate_anchor(desc);
    if (st != ATTN_OK) return -(int32_t)st;
    if (cu_count < 1) return -(int32_t)ATTN_ERR_VALUE;
    if (desc->num_blocks == 0) return 0;
    AnchorPlans a;
    if ((st = anchor_plans(desc, cu_count, true, &a)) != ATTN_OK) return -(int32_t)st;
    return a.fuse ? 1 : 0;
  } catch (...) {
    return -(int32_t)ATTN_ERR_HIP;
  }
}

attn_status_t attn_testing_plan(const attn_desc_t *desc, int32_t cu_count, attn_plan_t *plan) {
  try {
    if (!plan) return ATTN_ERR_NULL;
    return make_plan(desc, cu_count, true, plan);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_testing_check_decode(const attn_desc_t *desc, const attn_paged_kv_t *paged,
                                        const void *q, const void *k, const void *v,
                                        const float *o, const float *lse, int32_t need_v,
                                        int32_t need_o) {
  try {
    attn_status_t st = check_inputs(desc, q, k, v, need_v != 0);
    if (st != ATTN_OK) return st;
    if ((st = check_outputs(desc, o, lse, need_o != 0)) != ATTN_OK) return st;
    KvPaging pg;
    return validate_paged(desc, paged, &pg);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_testing_check_bifurcated(const attn_bifurcated_desc_t *desc, int32_t cu_count,
                                            size_t *workspace_bytes) {
  try {
    attn_status_t st = validate_bifurcated(desc);
    if (st != ATTN_OK) return st;
    if (!workspace_bytes) return ATTN_ERR_NULL;
    *workspace_bytes = 0;
    if (desc->num_samples == 0) return ATTN_OK;
    if (cu_count < 1) return ATTN_ERR_VALUE;
    BifPlans b;
    if ((st = bifurcated_plans(desc, cu_count, &b)) != ATTN_OK) return st;
    *workspace_bytes = b.total;
    return ATTN_OK;
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_testing_bifurcated_form(const attn_bifurcated_desc_t *desc, int32_t cu_count,
                                           int32_t *fused, int64_t *prefix_wgs,
                                           int64_t *suffix_wgs) {
  try {
    attn_status_t st = validate_bifurcated(desc);
    if (st != ATTN_OK) return st;
    if (!fused || !prefix_wgs || !suffix_wgs) return ATTN_ERR_NULL;
    *fused = 0;
    *prefix_wgs = *suffix_wgs = 0;
    if (desc->num_samples == 0) return ATTN_OK;
    if (cu_count < 1) return ATTN_ERR_VALUE;
    BifPlans b;
    if ((st = bifurcated_plans(desc, cu_count, &b)) != ATTN_OK) return st;
    *fused = b.fused ? 1 : 0;
    *prefix_wgs = work_map(&b.pre, b.pp).n_wg;
    *suffix_wgs = work_map(&b.suf, b.sp).n_wg;
    return ATTN_OK;
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

}  // extern "C"
