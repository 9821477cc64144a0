// The anchor-block prefill forced onto its three-launch path (anchor split,
// local split, merge), for tests that compare it with the single-merge path
// on shapes that take that one.  Linked into the test build of the library
// only.
#include "abi_internal.h"
#include "attn_decode_testing.h"

extern "C" attn_status_t attn_testing_prefill_anchor_unfused(
    const attn_anchor_desc_t *desc, const void *q, const void *k_anchor, const void *v_anchor,
    const void *k_blocks, const void *v_blocks, float *o, float *lse, void *workspace,
    size_t workspace_bytes, void *stream) {
  try {
    return attn::prefill_anchor_impl(desc, q, k_anchor, v_anchor, k_blocks, v_blocks, o, lse,
                                     workspace, workspace_bytes, stream, false);
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}
