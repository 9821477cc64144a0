// C-ABI entry points: validate on the host, partition, enqueue the split
// kernel(s) and the merge on the caller's stream.  Nothing here allocates,
// synchronises or keeps device state (the CU count per device is cached).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "attn_decode.h"
#include "abi_internal.h"
#include "kernels.h"
#include "plan.h"

namespace {

using namespace attn;

constexpr bool kMfma = true;  // dense query blocks go to the MFMA kernel
constexpr float kLog2eHost = 1.4426950408889634f;

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_cache[kMaxDevices];

attn_status_t device_cu_count(int *cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = g_cu_cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cu = c;
      return ATTN_OK;
    }
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1)
    return ATTN_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) g_cu_cache[dev].store(c, std::memory_order_relaxed);
  *cu = c;
  return ATTN_OK;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Lay the (m, l, o) records of a plan out in a workspace slice.
PartialLayout carve(char *base, const attn_plan_t &p, int head_dim) {
  PartialLayout pl{};
  pl.rows = p.rows_per_block;
  const int64_t records = p.record_slots * p.rows_per_block;
  if (records <= 0 || !base) return pl;
  const int64_t ml = round_up(records * (int64_t)sizeof(float), 256);
  pl.m = reinterpret_cast<float *>(base);
  pl.l = reinterpret_cast<float *>(base + ml);
  pl.o = reinterpret_cast<float *>(base + 2 * ml);
  (void)head_dim;
  return pl;
}

SplitArgs split_args(const attn_desc_t *d, const attn_plan_t &p, const void *q, const void *k,
                     const void *v, const void *zeta, const KvPaging &pg,
                     const PartialLayout &part) {
  SplitArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.zeta = zeta;
  a.pg = pg;
  a.map = work_map(d, p);
  a.part = part;
  a.q_len = d->q_len;
  a.Hq = d->num_q_heads;
  a.G = d->num_q_heads / d->num_kv_heads;
  a.R = p.rows;
  a.causal = d->causal;
  a.scale_log2 = d->scale * kLog2eHost;
  return a;
}

hipError_t launch_split(const attn_desc_t *d, const attn_plan_t &p, const SplitArgs &a,
                        SplitMode mode, hipStream_t s) {
  if (p.work_items <= 0) return hipSuccess;
  if (p.kernel >= 1) {
    if (mode == SplitMode::kEnergyZeta) return hipErrorInvalidValue;
    return launch_split_mfma(p, a, d->head_dim, mode == SplitMode::kEnergy, s);
  }
  return launch_split_valu(p, a, d->dtype, d->head_dim, mode, s);
}

// The energy at a given zeta runs on the vector-ALU kernel for every shape;
// everything else may use the MFMA kernels.
bool mfma_for(SplitMode mode) { return kMfma && mode != SplitMode::kEnergyZeta; }

// Workspace every decode entry point accepts for a descriptor: the larger of
// the two plans' record areas.
attn_status_t workspace_need(const attn_desc_t *d, int cu, size_t *bytes) {
  attn_plan_t a, b;
  attn_status_t st;
  if ((st = make_plan(d, cu, kMfma, &a)) != ATTN_OK) return st;
  if ((st = make_plan(d, cu, false, &b)) != ATTN_OK) return st;
  *bytes = a.workspace_bytes > b.workspace_bytes ? a.workspace_bytes : b.workspace_bytes;
  return ATTN_OK;
}

// Shared preamble of the decode entry points: validate, plan, check the
// workspace.  Returns ATTN_OK with *empty set when there is nothing to do.
attn_status_t prepare(const attn_desc_t *d, bool mfma, void *ws, size_t ws_bytes, attn_plan_t *p,
                      PartialLayout *part, bool *empty) {
  *empty = false;
  attn_status_t st = validate_desc(d);
  if (st != ATTN_OK) return st;
  if (d->batch == 0) {
    *empty = true;
    return ATTN_OK;
  }
  int cu = 0;
  if ((st = device_cu_count(&cu)) != ATTN_OK) return st;
  if ((st = make_plan(d, cu, mfma, p)) != ATTN_OK) return st;
  if ((st = check_workspace(p->workspace_bytes, ws, ws_bytes)) != ATTN_OK) return st;
  *part = carve(static_cast<char *>(ws), *p, d->head_dim);
  return ATTN_OK;
}

// The split phase.  v == null in kFull mode means energy only (the public
// partials entry points take "no V" as "no o").
attn_status_t partials_impl(const attn_desc_t *d, const attn_paged_kv_t *paged, const void *q,
                            const void *k, const void *v, const void *zeta, SplitMode mode,
                            void *ws, size_t ws_bytes, void *stream) {
  KvPaging pg;
  attn_status_t st = validate_paged(d, paged, &pg);
  if (st != ATTN_OK) return st;
  attn_plan_t p;
  PartialLayout part;
  bool empty;
  if ((st = prepare(d, mfma_for(mode), ws, ws_bytes, &p, &part, &empty)) != ATTN_OK || empty)
    return st;
  (void)hipGetLastError();
  if (launch_split(d, p, split_args(d, p, q, k, v, zeta, pg, part), mode,
                   static_cast<hipStream_t>(stream)) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

attn_status_t merge_impl(const attn_desc_t *d, bool mfma, float *o, float *lse, void *ws,
                         size_t ws_bytes, void *stream) {
  attn_plan_t p;
  PartialLayout part;
  bool empty;
  attn_status_t st = prepare(d, mfma, ws, ws_bytes, &p, &part, &empty);
  if (st != ATTN_OK || empty) return st;
  MergeArgs m{};
  m.map = work_map(d, p);
  m.part = part;
  m.q_len = d->q_len;
  m.Hq = d->num_q_heads;
  m.G = d->num_q_heads / d->num_kv_heads;
  m.R = p.rows;
  m.o = o;
  m.lse = lse;
  (void)hipGetLastError();
  if (launch_merge(m, d->head_dim, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

attn_status_t decode_impl(const attn_desc_t *d, const attn_paged_kv_t *paged, const void *q,
                          const void *k, const void *v, const void *zeta, float *o, float *lse,
                          void *ws, size_t ws_bytes, void *stream, SplitMode mode) {
  const bool need_o = mode == SplitMode::kFull;
  attn_status_t st = check_inputs(d, q, k, v, mode != SplitMode::kEnergy);
  if (st != ATTN_OK) return st;
  if ((st = check_outputs(d, o, lse, need_o)) != ATTN_OK) return st;
  if (mode == SplitMode::kEnergyZeta) {
    if (d->batch > 0 && !zeta) return ATTN_ERR_NULL;
    if (!aligned(zeta, 16)) return ATTN_ERR_ALIGN;
  }
  if ((st = partials_impl(d, paged, q, k, need_o || mode == SplitMode::kEnergyZeta ? v : nullptr,
                          zeta, mode, ws, ws_bytes, stream)) != ATTN_OK)
    return st;
  return merge_impl(d, mfma_for(mode), need_o ? o : nullptr, lse, ws, ws_bytes, stream);
}

}  // namespace

extern "C" {

attn_status_t attn_decode_plan(const attn_desc_t *desc, int32_t cu_count, attn_plan_t *plan) {
  try {
    attn_status_t st = validate_desc(desc);
    if (st != ATTN_OK) return st;
    if (!plan) return ATTN_ERR_NULL;
    int cu = cu_count;
    if (cu <= 0 && (st = device_cu_count(&cu)) != ATTN_OK) return st;
    return make_plan(desc, cu, kMfma, plan);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_workspace_bytes(const attn_desc_t *desc, size_t *bytes) {
  try {
    attn_status_t st = validate_desc(desc);
    if (st != ATTN_OK) return st;
    if (!bytes) return ATTN_ERR_NULL;
    *bytes = 0;
    if (desc->batch == 0) return ATTN_OK;
    int cu = 0;
    if ((st = device_cu_count(&cu)) != ATTN_OK) return st;
    return workspace_need(desc, cu, bytes);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_decode_energy(const attn_desc_t *desc, const void *q, const void *k,
                                 float *lse, void *workspace, size_t workspace_bytes,
                                 void *stream) {
  try {
    return decode_impl(desc, nullptr, q, k, nullptr, nullptr, nullptr, lse, workspace,
                       workspace_bytes, stream, SplitMode::kEnergy);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_decode(const attn_desc_t *desc, const void *q, const void *k, const void *v,
                          float *o, float *lse, void *workspace, size_t workspace_bytes,
                          void *stream) {
  try {
    return decode_impl(desc, nullptr, q, k, v, nullptr, o, lse, workspace, workspace_bytes, stream,
                       SplitMode::kFull);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_decode_partials(const attn_desc_t *desc, const void *q, const void *k,
                                   const void *v, void *workspace, size_t workspace_bytes,
                                   void *stream) {
  try {
    attn_status_t st = check_inputs(desc, q, k, v, false);
    if (st != ATTN_OK) return st;
    return partials_impl(desc, nullptr, q, k, v, nullptr,
                         v ? SplitMode::kFull : SplitMode::kEnergy, workspace, workspace_bytes,
                         stream);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_decode_merge(const attn_desc_t *desc, float *o, float *lse, void *workspace,
                                size_t workspace_bytes, void *stream) {
  try {
    attn_status_t st = check_outputs(desc, o, lse, false);
    if (st != ATTN_OK) return st;
    return merge_impl(desc, kMfma, o, lse, workspace, workspace_bytes, stream);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_decode_energy_zeta(const attn_desc_t *desc, const void *q, const void *k,
                                      const void *v, const void *zeta, float *lse,
                                      void *workspace, size_t workspace_bytes, void *stream) {
  try {
    return decode_impl(desc, nullptr, q, k, v, zeta, nullptr, lse, workspace, workspace_bytes,
                       stream, SplitMode::kEnergyZeta);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_decode_paged(const attn_desc_t *desc, const attn_paged_kv_t *paged,
                                const void *q, const void *k_pool, const void *v_pool, float *o,
                                float *lse, void *workspace, size_t workspace_bytes,
                                void *stream) {
  try {
    if (!paged) return ATTN_ERR_NULL;
    return decode_impl(desc, paged, q, k_pool, v_pool, nullptr, o, lse, workspace,
                       workspace_bytes, stream, SplitMode::kFull);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_decode_energy_paged(const attn_desc_t *desc, const attn_paged_kv_t *paged,
                                       const void *q, const void *k_pool, float *lse,
                                       void *workspace, size_t workspace_bytes, void *stream) {
  try {
    if (!paged) return ATTN_ERR_NULL;
    return decode_impl(desc, paged, q, k_pool, nullptr, nullptr, nullptr, lse, workspace,
                       workspace_bytes, stream, SplitMode::kEnergy);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_decode_partials_paged(const attn_desc_t *desc, const attn_paged_kv_t *paged,
                                         const void *q, const void *k_pool, const void *v_pool,
                                         void *workspace, size_t workspace_bytes, void *stream) {
  try {
    if (!paged) return ATTN_ERR_NULL;
    attn_status_t st = check_inputs(desc, q, k_pool, v_pool, false);
    if (st != ATTN_OK) return st;
    return partials_impl(desc, paged, q, k_pool, v_pool, nullptr,
                         v_pool ? SplitMode::kFull : SplitMode::kEnergy, workspace,
                         workspace_bytes, stream);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_bifurcated_workspace_bytes(const attn_bifurcated_desc_t *desc, size_t *bytes) {
  try {
    attn_status_t st = validate_bifurcated(desc);
    if (st != ATTN_OK) return st;
    if (!bytes) return ATTN_ERR_NULL;
    *bytes = 0;
    if (desc->num_samples == 0) return ATTN_OK;
    int cu = 0;
    if ((st = device_cu_count(&cu)) != ATTN_OK) return st;
    BifPlans b;
    if ((st = bifurcated_plans(desc, cu, &b)) != ATTN_OK) return st;
    *bytes = b.total;
    return ATTN_OK;
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_decode_bifurcated(const attn_bifurcated_desc_t *desc, const void *q,
                                     const void *k_prefix, const void *v_prefix,
                                     const void *k_suffix, const void *v_suffix, float *o,
                                     float *lse, void *workspace, size_t workspace_bytes,
                                     void *stream) {
  try {
    attn_status_t st = validate_bifurcated(desc);
    if (st != ATTN_OK) return st;
    if (!q || !o || !lse || (desc->prefix_len > 0 && (!k_prefix || !v_prefix)) ||
        (desc->suffix_len > 0 && (!k_suffix || !v_suffix)))
      return ATTN_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k_prefix, 16) || !aligned(v_prefix, 16) ||
        !aligned(k_suffix, 16) || !aligned(v_suffix, 16) || !aligned(o, 4) || !aligned(lse, 4))
      return ATTN_ERR_ALIGN;
    if (desc->num_samples == 0) return ATTN_OK;
    int cu = 0;
    if ((st = device_cu_count(&cu)) != ATTN_OK) return st;
    BifPlans b;
    if ((st = bifurcated_plans(desc, cu, &b)) != ATTN_OK) return st;
    if ((st = check_workspace(b.total, workspace, workspace_bytes)) != ATTN_OK) return st;
    char *ws = static_cast<char *>(workspace);
    const PartialLayout pre = carve(ws, b.pp, desc->head_dim);
    const PartialLayout suf = carve(ws + b.pre_bytes, b.sp, desc->head_dim);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const SplitArgs pa = split_args(&b.pre, b.pp, q, k_prefix, v_prefix, nullptr,
                                    dense_paging(&b.pre), pre);
    const SplitArgs sa = split_args(&b.suf, b.sp, q, k_suffix, v_suffix, nullptr,
                                    dense_paging(&b.suf), suf);
    (void)hipGetLastError();
    if (b.fused) {
      if (launch_bifurcated(pa, sa, desc->head_dim, b.sp.rows_per_block, b.workgroups, s) !=
          hipSuccess)
        return ATTN_ERR_HIP;
    } else {
      if (launch_split(&b.pre, b.pp, pa, SplitMode::kFull, s) != hipSuccess) return ATTN_ERR_HIP;
      if (launch_split(&b.suf, b.sp, sa, SplitMode::kFull, s) != hipSuccess) return ATTN_ERR_HIP;
    }
    MergeArgs m{};
    m.map = work_map(&b.suf, b.sp);
    m.part = suf;
    m.has_shared = b.pp.work_items > 0;
    m.smap = work_map(&b.pre, b.pp);
    m.shared = pre;
    m.q_len = 1;
    m.Hq = desc->num_q_heads;
    m.G = desc->num_q_heads / desc->num_kv_heads;
    m.R = m.G;
    m.o = o;
    m.lse = lse;
    if (launch_merge(m, desc->head_dim, s) != hipSuccess) return ATTN_ERR_HIP;
    return ATTN_OK;
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_anchor_workspace_bytes(const attn_anchor_desc_t *desc, size_t *bytes) {
  try {
    attn_status_t st = validate_anchor(desc);
    if (st != ATTN_OK) return st;
    if (!bytes) return ATTN_ERR_NULL;
    *bytes = 0;
    if (desc->num_blocks == 0) return ATTN_OK;
    int cu = 0;
    if ((st = device_cu_count(&cu)) != ATTN_OK) return st;
    AnchorPlans a;
    if ((st = anchor_plans(desc, cu, true, &a)) != ATTN_OK) return st;
    *bytes = a.total;
    return ATTN_OK;
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

attn_status_t attn_prefill_anchor(const attn_anchor_desc_t *desc, const void *q,
                                  const void *k_anchor, const void *v_anchor,
                                  const void *k_blocks, const void *v_blocks, float *o,
                                  float *lse, void *workspace, size_t workspace_bytes,
                                  void *stream) {
  try {
    return prefill_anchor_impl(desc, q, k_anchor, v_anchor, k_blocks, v_blocks, o, lse,
                               workspace, workspace_bytes, stream, true);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

const char *attn_status_string(attn_status_t status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is null";
    case ATTN_ERR_SHAPE: return "a size is out of range, or num_q_heads % num_kv_heads != 0";
    case ATTN_ERR_DTYPE: return "unknown element type";
    case ATTN_ERR_ALIGN: return "a tensor base pointer is misaligned";
    case ATTN_ERR_WORKSPACE: return "workspace smaller than the size query returned";
    case ATTN_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case ATTN_ERR_UNSUPPORTED: return "shape not covered by the kernels (head_dim must be 64 or 128)";
    case ATTN_ERR_VALUE: return "invalid scalar: non-finite scale, causal not 0/1, chunk_len "
                                "not a non-negative multiple of 64, or an invalid paging "
                                "description";
    case ATTN_ERR_SCRATCH: return "the call needs more record space than the static scratch "
                                  "array holds (ATTN_STATIC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

}  // extern "C"

namespace attn {

attn_status_t decode_with_workspace(const attn_desc_t *desc, const void *q, const void *k,
                                    const void *v, float *o, float *lse, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  return decode_impl(desc, nullptr, q, k, v, nullptr, o, lse, workspace, workspace_bytes, stream,
                     SplitMode::kFull);
}

// Anchor-block context encoding: the anchor part as one call over a cache
// shared by every block (sequence stride 0), the local part as a causal call
// over each block's own cache; both leave records for the same rows, merged
// by the merge kernel, or by the local call itself when every segment of
// both parts is one piece (fusion).
attn_status_t prefill_anchor_impl(const attn_anchor_desc_t *desc, const void *q,
                                  const void *k_anchor, const void *v_anchor,
                                  const void *k_blocks, const void *v_blocks, float *o,
                                  float *lse, void *workspace, size_t workspace_bytes,
                                  void *stream, bool allow_fusion) {
  attn_status_t st = validate_anchor(desc);
  if (st != ATTN_OK) return st;
  const bool any = desc->num_blocks > 0;
  if (any && (!q || !k_blocks || !v_blocks || !o || !lse ||
              (desc->anchor_len > 0 && (!k_anchor || !v_anchor))))
    return ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_anchor, 16) || !aligned(v_anchor, 16) ||
      !aligned(k_blocks, 16) || !aligned(v_blocks, 16) || !aligned(o, 4) || !aligned(lse, 4))
    return ATTN_ERR_ALIGN;
  if (!any) return ATTN_OK;
  int cu = 0;
  if ((st = device_cu_count(&cu)) != ATTN_OK) return st;
  AnchorPlans a;
  if ((st = anchor_plans(desc, cu, allow_fusion, &a)) != ATTN_OK) return st;
  if ((st = check_workspace(a.total, workspace, workspace_bytes)) != ATTN_OK) return st;
  char *ws = static_cast<char *>(workspace);
  const PartialLayout anc = carve(ws, a.ap, desc->head_dim);
  const PartialLayout loc = carve(ws + a.anc_bytes, a.lp, desc->head_dim);
  hipStream_t s = static_cast<hipStream_t>(stream);
  KvPaging shared = dense_paging(&a.anc);
  shared.seq_stride = 0;  // every block reads the one anchor
  (void)hipGetLastError();
  if (launch_split(&a.anc, a.ap, split_args(&a.anc, a.ap, q, k_anchor, v_anchor, nullptr, shared, anc),
                   SplitMode::kFull, s) != hipSuccess)
    return ATTN_ERR_HIP;
  SplitArgs la = split_args(&a.loc, a.lp, q, k_blocks, v_blocks, nullptr, dense_paging(&a.loc),
                            loc);
  if (a.fuse) {
    la.fin = 1;
    la.fin_map = work_map(&a.anc, a.ap);
    la.fin_part = anc;
    la.fin_o = o;
    la.fin_lse = lse;
  }
  if (launch_split(&a.loc, a.lp, la, SplitMode::kFull, s) != hipSuccess) return ATTN_ERR_HIP;
  if (a.fuse) return ATTN_OK;
  MergeArgs m{};
  m.map = work_map(&a.loc, a.lp);
  m.part = loc;
  m.has_shared = a.ap.work_items > 0;
  m.shared_same_rows = 1;
  m.smap = work_map(&a.anc, a.ap);
  m.shared = anc;
  m.q_len = desc->block_len;
  m.Hq = desc->num_q_heads;
  m.G = desc->num_q_heads / desc->num_kv_heads;
  m.R = a.lp.rows;
  m.o = o;
  m.lse = lse;
  if (launch_merge(m, desc->head_dim, s) != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

}  // namespace attn
