"""How the shared-prefix call launches (host planning, CPU): one launch of
both parts with the CUs split between them in proportion to their estimated
times (matrix-core flops of the prefix against the suffix's HBM bytes), the
shared form where one part would get less than a round of the eight XCDs,
and two separate launches where the prefix does not take the 256-row blocks.
The GPU tests run each form against the oracle."""
import ctypes

import pytest

from long_context_exact_split_amd import binding


def form(S, Hq, Hkv, D, Lp, Ls, cu=256):
    try:
        lib = binding.load_testing_library()
    except RuntimeError:
        pytest.skip("test build not built")
    d = binding.AttnBifDesc(num_samples=S, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                            prefix_len=Lp, suffix_len=Ls, scale=0.1, dtype=0)
    f, p, s = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
    st = lib.attn_testing_bifurcated_form(ctypes.byref(d), cu, ctypes.byref(f), ctypes.byref(p),
                                          ctypes.byref(s))
    assert st == 0, binding.STATUS.get(st, st)
    return f.value, p.value, s.value


def test_bench_batch_splits_the_cus_evenly():
    # 64 samples x 4 query heads per KV head over a 16384-token prefix: 17.2 GFLOP
    # (134 MB at 128 flop/B) against 134 MB of suffix K/V.
    assert form(64, 32, 8, 128, 16384, 512) == (1, 128, 128)


def test_long_suffix_gets_more_cus():
    f, p, s = form(64, 32, 8, 128, 4096, 2048)
    assert f == 1 and p + s == 256 and p % 8 == 0 and 8 <= p < s


def test_longer_prefix_gets_more_cus():
    f, p, s = form(64, 32, 8, 128, 65536, 512)
    assert f == 1 and p + s == 256 and p % 8 == 0 and p > s >= 8


def test_tiny_suffix_keeps_every_workgroup_on_both_parts():
    assert form(64, 32, 8, 128, 16384, 8) == (1, 256, 256)


def test_other_cu_counts():
    assert form(64, 32, 8, 128, 16384, 512, cu=304) == (1, 152, 152)
    assert form(64, 32, 8, 128, 16384, 512, cu=8)[1:] == (8, 8)  # too few CUs to split


def test_small_batches_take_two_launches():
    assert form(8, 32, 8, 128, 1000, 100)[0] == 0      # 32 rows per KV head
    assert form(64, 32, 8, 128, 1000, 0)[0] == 0       # no suffix
    assert form(64, 32, 8, 128, 0, 100)[0] == 0        # no prefix


def test_split_whose_shares_overflow_falls_back_to_the_shared_form():
    # 2048 samples with 2^20-token suffixes (2^34 suffix tokens in all) and a
    # 2^30-token prefix: the estimate gives the prefix all but 8 workgroups,
    # whose 2^31-token suffix shares do not fit the work map's 32-bit ranges;
    # on all 256 workgroups both parts' shares do.
    assert form(2048, 32, 8, 128, 1 << 30, 1 << 20) == (1, 256, 256)
    # half the samples (2^30-token suffix shares on 8 workgroups) split as estimated
    assert form(1024, 32, 8, 128, 1 << 30, 1 << 20)[1:] == (248, 8)
