"""Paged KV caches for the CPU oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

PagedAttention, as the "attention acceleration" concept page describes it in
its section 3, stores the KV cache in fixed-size blocks of tokens and keeps,
per sequence, a table that maps each logical block to a physical block, much
as virtual memory maps pages; blocks need not be contiguous and several
sequences may map the same physical block (a common prompt prefix).  Paging
changes where a token's key and value rows are stored, not what attention
computes, so the oracle resolves the mapping back into the dense logical
cache and then applies the plain definition (``attention.attend``).

Addressing (element offsets into a flat pool; P tokens per page):
    row(b, kvh, t) = table[b][t // P] * page_stride + kvh * head_stride
                     + (t % P) * token_stride,      elements row .. row + D - 1
Only tokens t < kv_lens[b] are resolved; the rest of the dense result is NaN,
so a reader of a position that the method never reads sees a poisoned value.
"""
from __future__ import annotations

import numpy as np

from .attention import attend


def gather(pool: np.ndarray, table: np.ndarray, kv_lens, page_size: int, page_stride: int,
           head_stride: int, token_stride: int, Hkv: int, D: int, L_max: int) -> np.ndarray:
    """Dense [B][Hkv][L_max][D] copy of a paged cache (NaN past each length)."""
    pool = np.asarray(pool).reshape(-1)
    table = np.asarray(table, dtype=np.int64)
    lens = np.asarray(kv_lens, dtype=np.int64).reshape(-1)
    B = lens.shape[0]
    nan = np.uint16(0x7FC0) if pool.dtype == np.uint16 else np.float32(np.nan)
    out = np.full((B, Hkv, L_max, D), nan, dtype=pool.dtype)
    cols = np.arange(D, dtype=np.int64)
    step = 1 << 16
    for b in range(B):
        for t0 in range(0, int(lens[b]), step):
            t = np.arange(t0, min(int(lens[b]), t0 + step), dtype=np.int64)
            page = table[b, t // page_size]
            if (page < 0).any():
                raise ValueError(f"sequence {b}: a visible token maps to no page")
            for kvh in range(Hkv):
                row = page * page_stride + kvh * head_stride + (t % page_size) * token_stride
                out[b, kvh, t0:t0 + t.size] = pool[row[:, None] + cols[None, :]]
    return out


def attend_paged(q, k_pool, v_pool, table, kv_lens, scale, *, page_size, page_stride,
                 head_stride, token_stride, num_kv_heads, L_max, causal=False, rows=None):
    """Plain attention over a paged cache: (O or None, lse) as ``attend`` returns
    them.  ``v_pool`` None gives the logsumexp only."""
    D = q.shape[-1]
    geo = (page_size, page_stride, head_stride, token_stride, num_kv_heads, D, L_max)
    k = gather(k_pool, table, kv_lens, *geo)
    v = None if v_pool is None else gather(v_pool, table, kv_lens, *geo)
    return attend(q, k, v, kv_lens, scale, causal=causal, rows=rows)
