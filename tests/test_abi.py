"""C-ABI boundary on the CPU: symbols, struct layout, validation errors.

Every call here fails validation, or is a pure-host plan query, or (valid
descriptors) is given a 1-byte workspace: no kernel is ever launched, even
where a GPU is visible, and none is needed."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from long_context_exact_split_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_decode.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        pytest.skip("library not built")
    return binding.load_library()


def declared_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def all_declared_functions():
    import glob
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        names.update(declared_functions(h))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    assert "attn_testing_pieces" not in names  # the testing hook has its own header
    for n in ("attn_decode_energy", "attn_decode", "attn_decode_bifurcated"):
        assert n in names
    assert set(names) == set(binding.EXPORTS)


def exported_functions(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    return set(re.findall(r"\bT (\S+)$", out, flags=re.M))


def test_library_exports_exactly_the_declared_boundary(lib):
    exported = exported_functions(binding.library_path())
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    # Nothing else: no test hook, no internal C++ symbol.
    assert exported == set(declared_functions()), sorted(exported - set(declared_functions()))


def test_testing_library_exports_its_hooks_and_the_boundary(lib):
    path = os.path.join(os.path.dirname(binding.library_path()), binding.TESTING_LIB_NAME)
    if not os.path.exists(path):
        pytest.skip("test build not built")
    exported = exported_functions(path)
    hooks = declared_functions(os.path.join(ROOT, "include", "attn_decode_testing.h"))
    assert "attn_testing_pieces" in hooks
    assert exported == set(all_declared_functions()), sorted(exported ^ set(all_declared_functions()))


def test_stamping_build_exports_the_boundary_and_its_probe(lib):
    """The bench's per-workgroup timing build: the same boundary plus the
    stamp read-back, which the product library does not have."""
    from long_context_exact_split_amd import build
    path = os.path.join(build.PKG, build.STAMPS_LIB_NAME)
    if not os.path.exists(path):
        pytest.skip("stamping build not built")
    exported = exported_functions(path)
    probes = {"attn_probe_wg_stamps", "attn_probe_wg_stamps_mfma", "attn_probe_wg_stamps_bif"}
    assert exported == set(declared_functions()) | probes
    assert not probes & exported_functions(binding.library_path())


def test_struct_layouts_match_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "attn_decode.h"
#define F(T, m) printf(#T "." #m " %zu\\n", offsetof(T, m));
int main(void) {
  printf("attn_desc_t %zu\\n", sizeof(attn_desc_t));
  F(attn_desc_t, max_kv_len) F(attn_desc_t, kv_lens) F(attn_desc_t, scale)
  F(attn_desc_t, chunk_len) F(attn_desc_t, dtype)
  printf("attn_plan_t %zu\\n", sizeof(attn_plan_t));
  F(attn_plan_t, balanced) F(attn_plan_t, threads_per_item) F(attn_plan_t, work_items)
  F(attn_plan_t, record_slots) F(attn_plan_t, cu_count) F(attn_plan_t, workspace_bytes)
  printf("attn_bifurcated_desc_t %zu\\n", sizeof(attn_bifurcated_desc_t));
  F(attn_bifurcated_desc_t, prefix_len) F(attn_bifurcated_desc_t, scale) F(attn_bifurcated_desc_t, dtype)
  printf("attn_anchor_desc_t %zu\\n", sizeof(attn_anchor_desc_t));
  F(attn_anchor_desc_t, head_dim) F(attn_anchor_desc_t, anchor_len) F(attn_anchor_desc_t, scale)
  F(attn_anchor_desc_t, dtype)
  printf("attn_paged_kv_t %zu\\n", sizeof(attn_paged_kv_t));
  F(attn_paged_kv_t, pages_per_seq) F(attn_paged_kv_t, page_size) F(attn_paged_kv_t, num_pages)
  F(attn_paged_kv_t, page_stride) F(attn_paged_kv_t, head_stride) F(attn_paged_kv_t, token_stride)
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = dict(line.rsplit(" ", 1) for line in subprocess.run([str(exe)], capture_output=True,
                                                               text=True, check=True).stdout.split("\n") if line)
    structs = {"attn_desc_t": binding.AttnDesc, "attn_plan_t": binding.AttnPlan,
               "attn_bifurcated_desc_t": binding.AttnBifDesc, "attn_paged_kv_t": binding.AttnPagedKv,
               "attn_anchor_desc_t": binding.AttnAnchorDesc}
    for key, val in got.items():
        if "." in key:
            s, f = key.split(".")
            assert getattr(structs[s], f).offset == int(val), key
        else:
            assert ctypes.sizeof(structs[key]) == int(val), key


def _desc(**kw):
    base = dict(batch=2, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=128, max_kv_len=1000)
    base.update(kw)
    return binding.make_desc(**base)


BAD = [
    (dict(num_q_heads=6, num_kv_heads=4), "ATTN_ERR_SHAPE"),
    (dict(q_len=0), "ATTN_ERR_SHAPE"),
    (dict(batch=-1), "ATTN_ERR_SHAPE"),
    (dict(max_kv_len=-5), "ATTN_ERR_SHAPE"),
    (dict(max_kv_len=2 ** 31), "ATTN_ERR_SHAPE"),
    # token indices stay in int32 with the kernels' read-ahead: at most 2^31 - 2^16
    (dict(max_kv_len=2 ** 31 - 2 ** 16 + 1), "ATTN_ERR_SHAPE"),
    (dict(max_kv_len=2 ** 31 - 1), "ATTN_ERR_SHAPE"),
    (dict(max_kv_len=2 ** 31 - 2 ** 16), None),  # valid: the largest extent
    (dict(num_kv_heads=0), "ATTN_ERR_SHAPE"),
    (dict(head_dim=96), "ATTN_ERR_UNSUPPORTED"),
    (dict(head_dim=0), "ATTN_ERR_SHAPE"),
    (dict(dtype=7), "ATTN_ERR_DTYPE"),
    (dict(scale=float("nan")), "ATTN_ERR_VALUE"),
    (dict(scale=float("inf")), "ATTN_ERR_VALUE"),
    (dict(chunk_len=100), "ATTN_ERR_VALUE"),
    (dict(chunk_len=-64), "ATTN_ERR_VALUE"),
    (dict(causal=True), None),  # valid
]


@pytest.mark.parametrize("kw,status", BAD)
def test_validation_errors_before_any_hip_call(lib, kw, status):
    d = _desc(**kw)
    code = lib.attn_decode(ctypes.byref(d), 16, 16, 16, 16, 16, 16, 1, None)
    e = lib.attn_decode_energy(ctypes.byref(d), 16, 16, 16, 16, 1, None)
    if status is None:
        # ATTN_ERR_HIP without a GPU, ATTN_ERR_WORKSPACE with one
        assert code in (5, 6) and e in (5, 6)
        return
    assert binding.STATUS[code] == status and binding.STATUS[e] == status


def test_null_and_alignment_errors(lib):
    d = _desc()
    assert binding.STATUS[lib.attn_decode(None, 16, 16, 16, 16, 16, 16, 1, None)] == "ATTN_ERR_NULL"
    assert binding.STATUS[lib.attn_decode(ctypes.byref(d), 0, 16, 16, 16, 16, 16, 1, None)] == "ATTN_ERR_NULL"
    assert binding.STATUS[lib.attn_decode(ctypes.byref(d), 16, 16, 0, 16, 16, 16, 1, None)] == "ATTN_ERR_NULL"
    assert binding.STATUS[lib.attn_decode(ctypes.byref(d), 16, 16, 16, 0, 16, 16, 1, None)] == "ATTN_ERR_NULL"
    # energy needs neither v nor o
    assert binding.STATUS[lib.attn_decode_energy(ctypes.byref(d), 16, 16, 0, 16, 1, None)] == "ATTN_ERR_NULL"
    assert binding.STATUS[lib.attn_decode(ctypes.byref(d), 8, 16, 16, 16, 16, 16, 1, None)] == "ATTN_ERR_ALIGN"
    assert binding.STATUS[lib.attn_decode(ctypes.byref(d), 16, 16, 16, 18, 16, 16, 1, None)] == "ATTN_ERR_ALIGN"
    # an empty batch is a valid no-op (no device needed)
    e = _desc(batch=0)
    assert lib.attn_decode(ctypes.byref(e), 16, 16, 16, 16, 16, 0, 0, None) == 0


def test_bifurcated_validation(lib):
    d = binding.AttnBifDesc()
    d.num_samples, d.num_q_heads, d.num_kv_heads, d.head_dim = 4, 8, 2, 128
    d.prefix_len, d.suffix_len, d.scale, d.dtype = 100, 10, 0.1, binding.ATTN_BF16
    args = [16] * 7 + [16, 1, None]
    d.num_q_heads = 7
    assert binding.STATUS[lib.attn_decode_bifurcated(ctypes.byref(d), *args)] == "ATTN_ERR_SHAPE"
    d.num_q_heads = 8
    d.dtype = binding.ATTN_F32
    assert binding.STATUS[lib.attn_decode_bifurcated(ctypes.byref(d), *args)] == "ATTN_ERR_UNSUPPORTED"
    d.dtype = binding.ATTN_BF16
    d.head_dim = 80
    assert binding.STATUS[lib.attn_decode_bifurcated(ctypes.byref(d), *args)] == "ATTN_ERR_UNSUPPORTED"
    d.head_dim = 128
    d.suffix_len = -1
    assert binding.STATUS[lib.attn_decode_bifurcated(ctypes.byref(d), *args)] == "ATTN_ERR_SHAPE"
    d.suffix_len = 2 ** 31 - 2 ** 16 + 1
    assert binding.STATUS[lib.attn_decode_bifurcated(ctypes.byref(d), *args)] == "ATTN_ERR_SHAPE"
    d.suffix_len = 10
    d.prefix_len = 2 ** 31 - 2 ** 16 + 1
    assert binding.STATUS[lib.attn_decode_bifurcated(ctypes.byref(d), *args)] == "ATTN_ERR_SHAPE"
    d.prefix_len = 100
    assert binding.STATUS[lib.attn_decode_bifurcated(ctypes.byref(d), *([16] * 6 + [0, 16, 1, None]))] == "ATTN_ERR_NULL"
    d.num_samples = 0
    assert lib.attn_decode_bifurcated(ctypes.byref(d), *args) == 0


def _paged(**kw):
    # head-major pages of 16 tokens for Hkv=2, D=128: page 4096 elements
    pk = binding.AttnPagedKv()
    base = dict(block_table=64, pages_per_seq=63, page_size=16, num_pages=200, page_stride=4096,
                head_stride=2048, token_stride=128)
    base.update(kw)
    for k, v in base.items():
        setattr(pk, k, v)
    return pk


BAD_PAGED = [
    (dict(page_size=12), "ATTN_ERR_VALUE"),
    (dict(page_size=0), "ATTN_ERR_VALUE"),
    (dict(page_size=1 << 21, pages_per_seq=1), "ATTN_ERR_VALUE"),
    (dict(pages_per_seq=62), "ATTN_ERR_VALUE"),   # 62 * 16 < max_kv_len = 1000
    (dict(pages_per_seq=0), "ATTN_ERR_VALUE"),
    (dict(num_pages=0), "ATTN_ERR_VALUE"),
    (dict(num_pages=-1), "ATTN_ERR_VALUE"),
    (dict(token_stride=-128), "ATTN_ERR_VALUE"),
    (dict(page_stride=1 << 40, num_pages=1 << 10), "ATTN_ERR_VALUE"),
    (dict(block_table=None), "ATTN_ERR_NULL"),
    (dict(token_stride=100), "ATTN_ERR_ALIGN"),   # rows must start on 16 bytes
    (dict(head_stride=2044), "ATTN_ERR_ALIGN"),
    (dict(page_size=1, pages_per_seq=1000), None),
    (dict(), None),
]


@pytest.mark.parametrize("kw,status", BAD_PAGED)
def test_paged_validation_before_any_hip_call(lib, kw, status):
    d = _desc()
    pk = _paged(**kw)
    codes = [lib.attn_decode_paged(ctypes.byref(d), ctypes.byref(pk), 16, 16, 16, 16, 16, 16,
                                   1, None),
             lib.attn_decode_energy_paged(ctypes.byref(d), ctypes.byref(pk), 16, 16, 16, 16,
                                          1, None),
             lib.attn_decode_partials_paged(ctypes.byref(d), ctypes.byref(pk), 16, 16, 16, 16,
                                            1, None)]
    for code in codes:
        if status is None:
            assert code not in (1, 2, 3, 4, 7, 8)  # may be ATTN_ERR_HIP without a GPU
        else:
            assert binding.STATUS[code] == status, (kw, code)


def test_paged_and_zeta_null_checks(lib):
    d = _desc()
    assert binding.STATUS[lib.attn_decode_paged(ctypes.byref(d), None, 16, 16, 16, 16, 16, 16,
                                                1, None)] == "ATTN_ERR_NULL"
    # fp32 pools need 16-byte rows too: 4-element multiples
    f = _desc(dtype=binding.ATTN_F32)
    pk = _paged(token_stride=132, head_stride=16 * 132, page_stride=2 * 16 * 132)
    assert lib.attn_decode_paged(ctypes.byref(f), ctypes.byref(pk), 16, 16, 16, 16, 16, 16,
                                 1, None) not in (1, 2, 3, 4, 7, 8)
    args = [16, 16, 16, 16, 16, 16, 1, None]
    assert binding.STATUS[lib.attn_decode_energy_zeta(ctypes.byref(d), *args)] not in (
        "ATTN_ERR_NULL", "ATTN_ERR_ALIGN")
    z = list(args); z[3] = 0
    assert binding.STATUS[lib.attn_decode_energy_zeta(ctypes.byref(d), *z)] == "ATTN_ERR_NULL"
    z[3] = 24
    assert binding.STATUS[lib.attn_decode_energy_zeta(ctypes.byref(d), *z)] == "ATTN_ERR_ALIGN"
    z = list(args); z[2] = 0  # F(zeta) reads V
    assert binding.STATUS[lib.attn_decode_energy_zeta(ctypes.byref(d), *z)] == "ATTN_ERR_NULL"


def test_anchor_validation(lib):
    d = binding.AttnAnchorDesc()
    d.num_blocks, d.block_len, d.num_q_heads, d.num_kv_heads, d.head_dim = 2, 64, 8, 2, 128
    d.anchor_len, d.scale, d.dtype = 100, 0.1, binding.ATTN_BF16
    args = [16] * 7 + [16, 1, None]

    def st(*a):
        return binding.STATUS[lib.attn_prefill_anchor(ctypes.byref(d), *(a or args))]
    d.num_q_heads = 7
    assert st() == "ATTN_ERR_SHAPE"
    d.num_q_heads = 8
    d.block_len = 0
    assert st() == "ATTN_ERR_SHAPE"
    d.block_len = 20000  # 4 x 20000 rows per KV head
    assert st() == "ATTN_ERR_UNSUPPORTED"
    d.block_len = 64
    d.dtype = binding.ATTN_F32
    assert st() == "ATTN_ERR_UNSUPPORTED"
    d.dtype = binding.ATTN_BF16
    d.anchor_len = -1
    assert st() == "ATTN_ERR_SHAPE"
    d.anchor_len = 2 ** 31 - 2 ** 16 + 1
    assert st() == "ATTN_ERR_SHAPE"
    d.anchor_len = 100
    assert st(*([16] * 3 + [0] + [16] * 4 + [1, None])) == "ATTN_ERR_NULL"   # k_blocks
    assert st(*([16] * 5 + [18] + [16] * 2 + [1, None])) == "ATTN_ERR_ALIGN"  # o not 4-byte aligned
    assert st(*([16] * 3 + [24] + [16] * 4 + [1, None])) == "ATTN_ERR_ALIGN"  # k_blocks not 16-byte
    d.anchor_len = 0  # no anchor: its tensors may be null
    assert st(*([16, 0, 0] + [16] * 5 + [1, None])) not in ("ATTN_ERR_NULL", "ATTN_ERR_ALIGN")
    d.num_blocks = 0
    assert lib.attn_prefill_anchor(ctypes.byref(d), *args) == 0


def test_merge_results_validation(lib):
    """attn_merge_results rejects bad sizes, null and misaligned pointers on
    the host; an empty call is a valid no-op that needs no device."""
    f = lib.attn_merge_results
    ok = [16, 16, 16, 16, None]
    assert binding.STATUS[f(0, 10, 128, *ok)] == "ATTN_ERR_SHAPE"
    assert binding.STATUS[f(-1, 10, 128, *ok)] == "ATTN_ERR_SHAPE"
    assert binding.STATUS[f(2, -1, 128, *ok)] == "ATTN_ERR_SHAPE"
    assert binding.STATUS[f(2, (1 << 25) + 1, 128, *ok)] == "ATTN_ERR_SHAPE"
    assert binding.STATUS[f(2, 10, 96, *ok)] == "ATTN_ERR_UNSUPPORTED"
    for i in range(4):
        args = list(ok)
        args[i] = 0
        assert binding.STATUS[f(2, 10, 64, *args)] == "ATTN_ERR_NULL"
        args[i] = 18
        assert binding.STATUS[f(2, 10, 64, *args)] == "ATTN_ERR_ALIGN"
    assert f(3, 0, 128, 0, 0, 0, 0, None) == 0
    # lse only takes both o_parts and o NULL; one of them NULL is an error
    assert binding.STATUS[f(2, 10, 64, 0, 16, 16, 16, None)] == "ATTN_ERR_NULL"
    assert binding.STATUS[f(2, 10, 64, 16, 16, 0, 16, None)] == "ATTN_ERR_NULL"
    assert binding.STATUS[f(2, 10, 64, 0, 0, 0, 16, None)] == "ATTN_ERR_NULL"
    assert binding.STATUS[f(2, 10, 64, 0, 18, 0, 16, None)] == "ATTN_ERR_ALIGN"


def test_merge_binding_refuses_host_tensors(lib):
    """The binding checks the tensors it hands over as pointers: host tensors
    are refused before the library is called (a host pointer in a kernel
    would fault the GPU)."""
    import torch
    with pytest.raises(ValueError):
        binding.merge_results(torch.zeros(2, 3, 64), torch.zeros(2, 3))
    with pytest.raises(ValueError):
        binding.merge_energies(torch.zeros(2, 3))
    with pytest.raises(ValueError):
        binding.merge_results(torch.zeros(2, 3, 64), torch.zeros(2, 4))


def test_status_strings(lib):
    for code, name in binding.STATUS.items():
        s = lib.attn_status_string(code).decode()
        assert s and s != "unknown status", name
    assert lib.attn_status_string(99).decode() == "unknown status"
