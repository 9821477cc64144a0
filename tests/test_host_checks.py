"""The entry points' host checks, run on their own through the test build.

attn_testing_check_decode and attn_testing_check_bifurcated run the same
validation code the entry points run before any launch (plan.cpp).  Here
they must return exactly what the exported entry points return for the same
arguments, over the validation tables of the ABI tests, so the host
sanitizer test (which loads a sanitized build of that code) exercises every
branch the ABI tests do.  No kernel is launched.
"""
import ctypes
import os

import pytest

from long_context_exact_split_amd import binding
from test_abi import BAD, BAD_PAGED, _desc, _paged

STATUS = binding.STATUS


@pytest.fixture(scope="module")
def tlib():
    try:
        return binding.load_testing_library()
    except RuntimeError:
        pytest.skip("test build not built")


@pytest.fixture(scope="module")
def lib():
    if os.environ.get("ATTN_TESTING_LIB"):
        return None  # sanitizer run: the host checks alone
    if not os.path.exists(binding.library_path()):
        pytest.skip("library not built")
    return binding.load_library()


@pytest.mark.parametrize("kw,status", BAD)
def test_decode_checks_match_entry_points(tlib, lib, kw, status):
    d = _desc(**kw)
    got = tlib.attn_testing_check_decode(ctypes.byref(d), None, 16, 16, 16, 16, 16, 1, 1)
    if status is None:
        assert got == 0
        return
    assert STATUS[got] == status
    if lib is not None:
        assert got == lib.attn_decode(ctypes.byref(d), 16, 16, 16, 16, 16, 16, 1, None)


@pytest.mark.parametrize("kw,status", BAD_PAGED)
def test_paged_checks_match_entry_points(tlib, lib, kw, status):
    d = _desc()
    pk = _paged(**kw)
    got = tlib.attn_testing_check_decode(ctypes.byref(d), ctypes.byref(pk), 16, 16, 16, 16, 16,
                                         1, 1)
    assert got == (0 if status is None else [k for k, v in STATUS.items() if v == status][0])
    if lib is not None and status is not None:
        assert got == lib.attn_decode_paged(ctypes.byref(d), ctypes.byref(pk), 16, 16, 16, 16, 16,
                                            16, 1, None)


def test_null_and_alignment_checks(tlib):
    d = _desc()
    c = lambda *a: STATUS[tlib.attn_testing_check_decode(ctypes.byref(d), None, *a)]
    assert c(0, 16, 16, 16, 16, 1, 1) == "ATTN_ERR_NULL"
    assert c(16, 16, 0, 16, 16, 1, 1) == "ATTN_ERR_NULL"
    assert c(16, 16, 0, 0, 16, 0, 0) == "ATTN_OK"        # energy: no v, no o
    assert c(16, 16, 16, 16, 0, 1, 1) == "ATTN_ERR_NULL"  # lse
    assert c(8, 16, 16, 16, 16, 1, 1) == "ATTN_ERR_ALIGN"
    assert c(16, 16, 16, 18, 16, 1, 1) == "ATTN_ERR_ALIGN"
    e = _desc(batch=0)
    assert STATUS[tlib.attn_testing_check_decode(ctypes.byref(e), None, 0, 0, 0, 16, 16, 1, 1)] \
        == "ATTN_OK"


def bif(**kw):
    d = binding.AttnBifDesc()
    base = dict(num_samples=64, num_q_heads=32, num_kv_heads=8, head_dim=128, prefix_len=16384,
                suffix_len=512, scale=0.088, dtype=binding.ATTN_BF16)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(), "ATTN_OK"), (dict(num_samples=0), "ATTN_OK"), (dict(prefix_len=0), "ATTN_OK"),
    (dict(suffix_len=0), "ATTN_OK"), (dict(prefix_len=0, suffix_len=0), "ATTN_OK"),
    (dict(num_samples=16384, prefix_len=2 ** 20, suffix_len=3), "ATTN_OK"),
    (dict(num_samples=16, prefix_len=2 ** 31 - 2 ** 16, suffix_len=2 ** 31 - 2 ** 16), "ATTN_OK"),
    # a workgroup's share of the tokens would pass 2^31
    (dict(num_samples=16384, prefix_len=2 ** 31 - 2 ** 16, suffix_len=3), "ATTN_ERR_UNSUPPORTED"),
    (dict(num_samples=16385), "ATTN_ERR_UNSUPPORTED"),  # 4 x 16385 prefix rows per KV head
    (dict(prefix_len=2 ** 31 - 2 ** 16 + 1), "ATTN_ERR_SHAPE"),
    (dict(num_q_heads=7), "ATTN_ERR_SHAPE"), (dict(head_dim=96), "ATTN_ERR_UNSUPPORTED"),
    (dict(dtype=binding.ATTN_F32), "ATTN_ERR_UNSUPPORTED"), (dict(scale=float("nan")), "ATTN_ERR_VALUE"),
])
def test_bifurcated_checks(tlib, kw, status):
    n = ctypes.c_size_t(0)
    got = tlib.attn_testing_check_bifurcated(ctypes.byref(bif(**kw)), 256, ctypes.byref(n))
    assert STATUS[got] == status
    if status == "ATTN_OK" and kw.get("num_samples", 64) and (kw.get("prefix_len", 1) or kw.get("suffix_len", 1)):
        assert n.value > 0
