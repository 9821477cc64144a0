"""When attn_prefill_anchor finalises rows in its local split (CPU, host logic).

The finalising path needs every segment of the anchor part and of the local
part to be a single piece, so that each row has exactly one record of each.
The library decides this from the workgroups' first pieces; here the same
fact is checked through a different route, the merge's own enumeration of a
segment's record slots, for shapes that fuse and shapes that do not.
"""
import os

import pytest

from long_context_exact_split_amd import binding as B

# Under the host sanitizer test the plan comes from the sanitized host build.
host_plan = B.testing_plan if os.environ.get("ATTN_TESTING_LIB") else B.plan

CU = 256


def anchor_desc(N, Lb, Hq, Hkv, D, A):
    d = B.AttnAnchorDesc()
    d.num_blocks, d.block_len, d.num_q_heads, d.num_kv_heads, d.head_dim = N, Lb, Hq, Hkv, D
    d.anchor_len, d.scale, d.dtype = A, 0.1, 0
    return d


def part_descs(N, Lb, Hq, Hkv, D, A):
    """The two calls the anchor entry point makes: anchor part, local part."""
    out = []
    for L, causal in ((A, 0), (Lb, 1)):
        d = B.AttnDesc()
        d.batch, d.q_len, d.num_q_heads, d.num_kv_heads, d.head_dim = N, Lb, Hq, Hkv, D
        d.max_kv_len, d.kv_lens, d.scale, d.causal, d.chunk_len, d.dtype = L, None, 0.1, causal, 0, 0
        out.append(d)
    return out


def slot_counts(d):
    p = host_plan(d, CU)
    segs = d.batch * d.num_kv_heads * p["row_blocks"]
    return p, [B.testing_segment_slots(d, None, CU, s)[2] for s in range(segs)]


FUSED = [(2, 8192, 32, 8, 128, 8192), (1, 9, 8, 2, 128, 100), (1, 23, 16, 4, 128, 64),
         (2, 64, 32, 8, 128, 64), (1, 2048, 64, 8, 64, 512), (2, 40, 8, 2, 128, 50)]
UNFUSED = [(2, 10, 32, 4, 128, 500), (3, 100, 8, 2, 128, 77), (2, 64, 4, 4, 128, 0),
           (2, 7, 8, 2, 128, 300)]


@pytest.mark.parametrize("shape", FUSED)
def test_fused_shapes_have_one_record_per_segment(shape):
    assert B.testing_anchor_fuses(anchor_desc(*shape), CU)
    for d in part_descs(*shape):
        p, counts = slot_counts(d)
        assert p["kernel"] == 2 and p["balanced"] == 1
        assert counts and all(c == 1 for c in counts), counts[:20]


@pytest.mark.parametrize("shape", UNFUSED)
def test_unfused_shapes_fail_a_condition(shape):
    assert not B.testing_anchor_fuses(anchor_desc(*shape), CU)
    reasons = []
    for d in part_descs(*shape):
        p, counts = slot_counts(d)
        if p["kernel"] != 2 or p["work_items"] == 0 or any(c != 1 for c in counts):
            reasons.append(d.causal)
    assert reasons, "no condition of the finalising path fails, yet it is not taken"


def test_bad_arguments_are_refused():
    with pytest.raises(B.AttnError):
        B.testing_anchor_fuses(anchor_desc(2, 8192, 32, 8, 96, 8192), CU)
    with pytest.raises(B.AttnError):
        B.testing_anchor_fuses(anchor_desc(2, 8192, 32, 8, 128, 8192), 0)
