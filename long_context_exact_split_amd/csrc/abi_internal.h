// Internal entry points of the library shared with its test build (hidden
// symbols: not part of the exported C ABI).
#pragma once

#include <stddef.h>

#include "attn_decode.h"

namespace attn {

// attn_prefill_anchor with the choice of its single-merge path made by the
// caller: allow_fusion = false always runs anchor split, local split and
// merge, so a test can compare the two paths on shapes that fuse.
attn_status_t prefill_anchor_impl(const attn_anchor_desc_t *desc, const void *q,
                                  const void *k_anchor, const void *v_anchor,
                                  const void *k_blocks, const void *v_blocks, float *o,
                                  float *lse, void *workspace, size_t workspace_bytes,
                                  void *stream, bool allow_fusion);

// attn_decode on a given workspace (the static-scratch entry point passes
// the library's own array).
attn_status_t decode_with_workspace(const attn_desc_t *desc, const void *q, const void *k,
                                    const void *v, float *o, float *lse, void *workspace,
                                    size_t workspace_bytes, void *stream);

}  // namespace attn
