// Row addressing of the K/V caches inside the split kernels: dense caches,
// and paged ones ("attention acceleration" concept page, section 3,
// PagedAttention: fixed-size pages of tokens found through a per-sequence
// block table).  The page lookup is a separate step from the address so a
// kernel can issue the table loads for a tile well before the K/V loads that
// depend on them.
#pragma once

#include "kernels.h"

namespace attn {

template <bool PAGED, int D>
struct KvRows {
  const int32_t *bt;  // this sequence's block-table row (paged)
  int64_t origin;     // added once to the pool pointer: dense, first row of (b, kvh);
                      // paged, kvh * head_stride
  int64_t page_stride, token_stride, num_pages;
  int32_t shift, mask;

  __device__ __forceinline__ KvRows(const SplitArgs &a, int b, int kvh) {
    if constexpr (PAGED) {
      bt = a.pg.block_table + (int64_t)b * a.pg.pages_per_seq;
      origin = (int64_t)kvh * a.pg.head_stride;
      page_stride = a.pg.page_stride;
      token_stride = a.pg.token_stride;
      num_pages = a.pg.num_pages;
      shift = a.pg.page_shift;
      mask = (1 << a.pg.page_shift) - 1;
    } else {
      bt = nullptr;
      origin = (int64_t)b * a.pg.seq_stride + (int64_t)kvh * a.map.L_max * D;
      page_stride = token_stride = num_pages = 0;
      shift = mask = 0;
    }
  }

  // Physical page of token t (paged; a load from the block table).
  __device__ __forceinline__ int32_t lookup(int t) const {
    if constexpr (PAGED) return bt[t >> shift];
    return 0;
  }

  // Element offset of token t's row from pool + origin, given lookup(t).
  __device__ __forceinline__ int64_t offset(int t, int32_t page) const {
    if constexpr (PAGED) {
      const int64_t p = (page >= 0 && page < num_pages) ? page : 0;
      return p * page_stride + (int64_t)(t & mask) * token_stride;
    }
    return (int64_t)t * D;
  }
};

}  // namespace attn
