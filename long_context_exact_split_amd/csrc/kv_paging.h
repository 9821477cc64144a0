// Paging description handed to the split kernels (host and device code).
#pragma once

#include <stdint.h>

namespace attn {

// Where the K and V rows live.  Dense (block_table null): row (b, kvh, t) at
// element b*seq_stride + (kvh*L_max + t)*D, seq_stride normally Hkv*L_max*D
// (0: every sequence reads one shared cache).  Paged: token t of sequence b is slot
// t % P of physical page block_table[b*pages_per_seq + t/P], and its row
// starts at page*page_stride + kvh*head_stride + (t % P)*token_stride.
// Table entries outside [0, num_pages) are read as page 0.
struct KvPaging {
  const int32_t *block_table;
  int64_t seq_stride;  // dense: elements from one sequence's cache to the next
  int64_t num_pages;
  int64_t page_stride, head_stride, token_stride;  // elements
  int32_t pages_per_seq;
  int32_t page_shift;  // log2 P
};

}  // namespace attn
