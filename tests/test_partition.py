"""KV-chunk partitioner (pure host code, explicit CU count)."""
import math

import pytest
from hypothesis import given, settings, strategies as st

from long_context_exact_split_amd import binding


def plan(cu=256, **kw):
    base = dict(batch=1, q_len=1, num_q_heads=32, num_kv_heads=8, head_dim=128, max_kv_len=4096)
    base.update(kw)
    return binding.plan(binding.make_desc(**base), cu)


def test_forced_chunk_len_single_query_fp32():
    p = plan(num_q_heads=1, num_kv_heads=1, head_dim=64, max_kv_len=4096, chunk_len=512,
             dtype=binding.ATTN_F32)
    assert p["chunk_len"] == 512 and p["chunks_per_seq"] == 8 and p["work_items"] == 8
    assert p["kernel"] == 0 and p["rows"] == 1 and p["rows_per_block"] == 1


def test_dense_decode_gives_one_item_per_cu():
    # every sequence full: one contiguous chunk per CU
    p = plan(batch=8, max_kv_len=32768)
    assert p["rows"] == 4 and p["rows_per_block"] == 4 and p["row_blocks"] == 1
    assert p["work_items"] == 256 and p["chunk_len"] == 8192
    p = plan(max_kv_len=1 << 20)
    assert p["work_items"] == 256 and p["chunk_len"] == 32768
    p = plan(max_kv_len=5_120_000)
    assert 256 >= p["work_items"] > 240 and p["chunks_per_seq"] * p["chunk_len"] >= 5_120_000


def test_ragged_lengths_get_finer_chunks():
    # lengths on the device: the host plans on max_kv_len with ~4 items per CU
    p = plan(batch=16, num_q_heads=32, num_kv_heads=8, max_kv_len=131072, kv_lens_ptr=0x1000)
    assert p["work_items"] >= 4 * 256 * 0.9


def test_empty_and_tiny():
    p = plan(max_kv_len=0)
    assert p["chunks_per_seq"] == 0 and p["work_items"] == 0 and p["workspace_bytes"] == 0
    p = plan(max_kv_len=1)
    assert p["chunks_per_seq"] == 1 and p["chunk_len"] == 256


@settings(max_examples=200, deadline=None)
@given(B=st.integers(1, 32), Hkv=st.integers(1, 16), G=st.integers(1, 16), q_len=st.integers(1, 8),
       L=st.integers(0, 3_000_000), cu=st.sampled_from([1, 8, 80, 256, 304]),
       D=st.sampled_from([64, 128]))
def test_every_token_covered_once(B, Hkv, G, q_len, L, cu, D):
    p = plan(cu=cu, batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, q_len=q_len, head_dim=D,
             max_kv_len=L)
    R = G * q_len
    assert p["rows"] == R
    assert p["rows_per_block"] * p["row_blocks"] >= R
    assert p["rows_per_block"] * (p["row_blocks"] - 1) < R
    C, n = p["chunk_len"], p["chunks_per_seq"]
    assert C > 0 and C % 64 == 0
    # chunks [c*C, (c+1)*C) for c < n tile [0, L) exactly, with no empty chunk
    assert n == (math.ceil(L / C) if L else 0)
    assert n * C >= L and (n == 0 or (n - 1) * C < L)
    assert p["work_items"] == B * Hkv * p["row_blocks"] * n
    records = B * Hkv * n * p["row_blocks"] * p["rows_per_block"]
    assert p["workspace_bytes"] >= records * (D + 2) * 4
    if records:
        assert p["workspace_bytes"] <= records * (D + 2) * 4 + 3 * 256


def test_plan_rejects_invalid_descriptor():
    d = binding.make_desc(batch=1, q_len=1, num_q_heads=3, num_kv_heads=2, head_dim=64, max_kv_len=10)
    with pytest.raises(binding.AttnError):
        binding.plan(d, 256)
