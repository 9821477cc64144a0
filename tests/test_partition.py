"""KV partition (host code; the same work_map arithmetic the kernels run).

Checked here, with host-side lengths through the testing hook:
* every token of every (sequence, KV head, row block) segment is covered by
  exactly one piece, and no piece is empty;
* record slots are distinct and inside the workspace's slot count;
* the slots the merge enumerates for a segment are exactly its pieces' slots,
  in token order;
* the balanced layout gives every workgroup the same number of tokens (+-1).
"""
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from long_context_exact_split_amd import binding

# Under the host sanitizer test the plan comes from the sanitized host build.
host_plan = binding.testing_plan if os.environ.get("ATTN_TESTING_LIB") else binding.plan


def desc(**kw):
    base = dict(batch=1, q_len=1, num_q_heads=32, num_kv_heads=8, head_dim=128, max_kv_len=4096)
    base.update(kw)
    return binding.make_desc(**base)


def plan(cu=256, **kw):
    return host_plan(desc(**kw), cu)


def test_forced_chunk_len_single_query_fp32():
    p = plan(num_q_heads=1, num_kv_heads=1, head_dim=64, max_kv_len=4096, chunk_len=512,
             dtype=binding.ATTN_F32)
    assert p["balanced"] == 0 and p["chunk_len"] == 512 and p["chunks_per_seq"] == 8
    assert p["work_items"] == 8 and p["record_slots"] == 8
    assert p["kernel"] == 0 and p["rows"] == 1 and p["rows_per_block"] == 1


def test_dense_decode_gives_one_share_per_cu():
    p = plan(batch=8, max_kv_len=32768)
    assert p["balanced"] == 1 and p["work_items"] == 256 and p["chunk_len"] == 8192
    assert p["rows"] == 4 and p["rows_per_block"] == 4 and p["kernel"] == 0
    p = plan(max_kv_len=1 << 20)
    assert p["work_items"] == 256 and p["chunk_len"] == 32768
    assert p["record_slots"] == 256 + 8 - 1


def test_query_blocks_go_to_mfma():
    p = plan(batch=16, q_len=4, num_q_heads=64, num_kv_heads=8, max_kv_len=131072,
             causal=True, kv_lens_ptr=0x1000)
    assert p["kernel"] == 1 and p["rows"] == 32 and p["rows_per_block"] == 32
    p = plan(dtype=binding.ATTN_F32, q_len=4, num_q_heads=64, num_kv_heads=8)
    assert p["kernel"] == 0 and p["rows_per_block"] == 8 and p["row_blocks"] == 4


def test_short_shares_get_two_workgroups_per_cu():
    # 64 sequences x 8 KV heads x 512 tokens: 1024 tokens per CU
    p = plan(batch=64, max_kv_len=512)
    assert p["kernel"] == 0 and p["work_items"] == 512
    # the MFMA kernels keep one workgroup per CU
    p = plan(batch=64, q_len=4, num_q_heads=64, max_kv_len=512, causal=True)
    assert p["kernel"] == 1 and p["work_items"] == 256


def test_small_calls_use_fewer_workgroups():
    p = plan(num_q_heads=1, num_kv_heads=1, max_kv_len=4096)
    assert p["work_items"] == 16   # at least 256 tokens per workgroup
    p = plan(max_kv_len=0)
    assert p["work_items"] == 0 and p["workspace_bytes"] == 0


def segment_keys(d, p, L_b, rb):
    """Keys a segment of the layout covers: all L_b, or under a causal mask
    with several row blocks of the shared-tile kernel (balanced layout) the
    keys the block's last row sees (written out from the visibility rule
    t <= L_b - q_len + i)."""
    if not (p["balanced"] and d.causal and p["row_blocks"] > 1 and p["kernel"] == 2):
        return L_b
    G = d.num_q_heads // d.num_kv_heads
    last_row = min(p["rows"], (rb + 1) * p["rows_per_block"]) - 1
    return min(L_b, max(0, L_b - d.q_len + last_row // G + 1))


def check_cover(d, lens, cu):
    p = host_plan(d, cu)
    B, Hkv = d.batch, d.num_kv_heads
    rbk = p["row_blocks"]
    L = np.full(B, d.max_kv_len) if lens is None else np.minimum(np.maximum(lens, 0), d.max_kv_len)
    segs = B * Hkv * rbk
    seg_len = [segment_keys(d, p, int(L[s // (Hkv * rbk)]), s % rbk) for s in range(segs)]
    covered = {s: [] for s in range(segs)}
    slots = set()
    per_wg = []
    for w in range(p["work_items"]):
        pieces = binding.testing_pieces(d, lens, cu, w)
        per_wg.append(sum(t1 - t0 for (_, t0, t1, _) in pieces))
        for (s, t0, t1, slot) in pieces:
            assert 0 <= t0 < t1 <= seg_len[s], (s, t0, t1)
            assert 0 <= slot < p["record_slots"], (slot, p["record_slots"])
            assert slot not in slots
            slots.add(slot)
            covered[s].append((t0, t1, slot))
    for s in range(segs):
        iv = sorted(covered[s])
        Ls = seg_len[s]
        pos = 0
        for (t0, t1, _) in iv:
            assert t0 == pos
            pos = t1
        assert pos == Ls, (s, pos, Ls)
        first, stride, count = binding.testing_segment_slots(d, lens, cu, s)
        assert [first + k * stride for k in range(count)] == [slot for (_, _, slot) in iv]
    if p["balanced"] and p["work_items"]:
        assert max(per_wg) - min(per_wg) <= 1
    return p


@settings(max_examples=120, deadline=None)
@given(B=st.integers(1, 6), Hkv=st.integers(1, 4), G=st.integers(1, 9), q_len=st.integers(1, 5),
       L=st.integers(0, 5000), cu=st.sampled_from([1, 3, 8, 40, 256]),
       forced=st.sampled_from([0, 0, 64, 448]), seed=st.integers(0, 2 ** 31),
       ragged=st.booleans(), D=st.sampled_from([64, 128]))
def test_pieces_tile_every_segment_exactly_once(B, Hkv, G, q_len, L, cu, forced, seed, ragged, D):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, L + 1, size=B).astype(np.int32) if ragged else None
    if ragged and rng.random() < 0.3:
        lens[rng.integers(0, B)] = 0
    d = desc(batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, q_len=q_len, head_dim=D,
             max_kv_len=L, chunk_len=forced, kv_lens_ptr=0x1000 if ragged else 0,
             causal=q_len > 1)
    check_cover(d, lens, cu)


@settings(max_examples=150, deadline=None)
@given(B=st.integers(1, 4), Hkv=st.integers(1, 3), G=st.integers(1, 8), q_len=st.integers(1, 160),
       L=st.integers(0, 3000), cu=st.sampled_from([1, 5, 40, 256]), seed=st.integers(0, 2 ** 31),
       ragged=st.booleans(), dt=st.sampled_from([binding.ATTN_BF16, binding.ATTN_F32]))
def test_causal_row_blocks_get_only_visible_keys(B, Hkv, G, q_len, L, cu, seed, ragged, dt):
    """Causal query blocks spanning several row blocks (prefill-like): each
    segment covers exactly the keys its last row sees, the pieces still tile
    every segment once, and workgroups get equal shares of visible keys."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, L + 1, size=B).astype(np.int32) if ragged else None
    d = desc(batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, q_len=q_len, max_kv_len=L,
             kv_lens_ptr=0x1000 if ragged else 0, causal=True, dtype=dt)
    check_cover(d, lens, cu)


def test_anchor_prefill_local_part_is_balanced_over_visible_keys():
    """Causal prefill of 2 blocks of 8192 tokens (Hq=32, Hkv=8): 128 row
    blocks of 64 tokens per KV head, which see 64, 128, ..., 8192 keys."""
    d = desc(batch=2, q_len=8192, num_q_heads=32, num_kv_heads=8, max_kv_len=8192, causal=True)
    p = host_plan(d, 256)
    assert p["kernel"] == 2 and p["row_blocks"] == 128
    units = 2 * 8 * sum(64 * (rb + 1) for rb in range(128))
    per_wg = []
    for w in range(p["work_items"]):
        per_wg.append(sum(t1 - t0 for (_, t0, t1, _) in binding.testing_pieces(d, None, 256, w)))
    assert sum(per_wg) == units
    assert max(per_wg) - min(per_wg) <= 1
    # Zigzag order of the row blocks: every workgroup gets as many pieces
    # (each costs a pipeline start and a record write), not 4 here and 30 there.
    pieces = [len(binding.testing_pieces(d, None, 256, w)) for w in range(p["work_items"])]
    assert max(pieces) - min(pieces) <= 1


def test_ragged_70b_shape_is_balanced():
    rng = np.random.default_rng(5)
    lens = rng.integers(8192, 131072, endpoint=True, size=16).astype(np.int32)
    d = desc(batch=16, q_len=4, num_q_heads=64, num_kv_heads=8, max_kv_len=131072, causal=True,
             kv_lens_ptr=0x1000)
    p = check_cover(d, lens, 256)
    assert p["work_items"] == 256


def test_plan_rejects_invalid_descriptor():
    d = binding.make_desc(batch=1, q_len=1, num_q_heads=3, num_kv_heads=2, head_dim=64,
                          max_kv_len=10)
    with pytest.raises(binding.AttnError):
        host_plan(d, 256)


# Extremes of the descriptor: the longest cache the boundary accepts (2^31 -
# 2^16 tokens) and the most query rows per KV head (2^16), alone and together
# under a causal mask, where the closed-form row-block sums run on their
# largest arguments.
KMAX = 2 ** 31 - 2 ** 16
EXTREMES = [
    dict(batch=1, num_q_heads=8, num_kv_heads=8, q_len=1, max_kv_len=KMAX),
    dict(batch=3, num_q_heads=32, num_kv_heads=8, q_len=1, max_kv_len=KMAX, ragged=True),
    dict(batch=1, num_q_heads=4, num_kv_heads=1, q_len=16384, max_kv_len=16384, causal=True),
    dict(batch=1, num_q_heads=4, num_kv_heads=1, q_len=16384, max_kv_len=KMAX, causal=True),
    dict(batch=2, num_q_heads=6, num_kv_heads=1, q_len=5461, max_kv_len=KMAX // 2, causal=True,
         ragged=True),
    dict(batch=1, num_q_heads=2, num_kv_heads=1, q_len=32768, max_kv_len=40000, causal=True),
]


@pytest.mark.parametrize("shape", EXTREMES, ids=[str(i) for i in range(len(EXTREMES))])
def test_extreme_shapes_tile_exactly(shape):
    shape = dict(shape)
    ragged = shape.pop("ragged", False)
    lens = None
    if ragged:
        rng = np.random.default_rng(7)
        lens = rng.integers(shape["max_kv_len"] // 2, shape["max_kv_len"], endpoint=True,
                            size=shape["batch"]).astype(np.int32)
        lens[0] = shape["max_kv_len"]
    d = desc(kv_lens_ptr=0x1000 if ragged else 0, **shape)
    p = check_cover(d, lens, 256)
    assert p["rows"] == (shape["num_q_heads"] // shape["num_kv_heads"]) * shape["q_len"]


def test_share_beyond_int32_is_refused():
    """A workgroup's share of the layout is an int32 token count: a call whose
    segments hold more than 256 * (2^31 - 1) tokens in all is refused."""
    d = desc(batch=2, num_q_heads=12, num_kv_heads=2, q_len=5461, max_kv_len=KMAX, causal=True)
    with pytest.raises(binding.AttnError):
        host_plan(d, 256)
