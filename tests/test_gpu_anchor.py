"""Anchor-block context encoding (Star Attention, phase 1) on the GPU against
the fp64 oracle: every row for small shapes spanning all three kernels and
ragged tiles, sampled rows at the benchmark size, and the exact identity that
with two blocks the second block equals global causal attention."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import check_rows, dev, say
from long_context_exact_split_amd import binding, inputs

pytestmark = pytest.mark.gpu


def make(N, Lb, Hq, Hkv, D, A, seed):
    rng = np.random.default_rng(seed)
    bits = lambda *s: inputs.f32_to_bf16(rng.standard_normal(s, dtype=np.float32))
    return (bits(N, Lb, Hq, D), bits(Hkv, A, D), bits(Hkv, A, D), bits(N, Hkv, Lb, D),
            bits(N, Hkv, Lb, D))


ANCHOR = [
    # N, Lb, Hq, Hkv, D, A
    (1, 1, 8, 2, 128, 100),      # one token per block: 4 rows, vector ALUs
    (2, 7, 8, 2, 128, 300),      # 28 rows: MFMA query-block kernel
    (3, 100, 8, 2, 64, 64),      # 400 rows: shared-tile kernel, 2 row blocks
    (2, 300, 32, 8, 128, 777),   # 1200 rows, ragged tiles
    (2, 64, 4, 4, 128, 0),       # no anchor: causal within each block
    (1, 257, 16, 2, 128, 1000),  # 2056 rows
    (2, 10, 32, 4, 128, 500),    # 80 rows: one row block
]


@pytest.mark.parametrize("case", ANCHOR, ids=[f"N{c[0]}_Lb{c[1]}_Hq{c[2]}_Hkv{c[3]}_D{c[4]}_A{c[5]}" for c in ANCHOR])
def test_anchor_blocks_small(case):
    N, Lb, Hq, Hkv, D, A = case
    say(f"anchor case {case}")
    q, ka, va, kb, vb = make(N, Lb, Hq, Hkv, D, A, seed=Lb * 7 + A)
    scale = 1.0 / np.sqrt(D)
    O, lse = binding.prefill_anchor(dev(q), dev(ka), dev(va), dev(kb), dev(vb), scale=scale)
    torch.cuda.synchronize()
    Or, lr = oracle.attend_anchor_blocks(q, ka, va, kb, vb, scale)
    check_rows(O.cpu().numpy(), lse.cpu().numpy(), Or, lr, what=f"anchor {case}")


def test_two_blocks_equal_global_causal_attention():
    """Block 1 with block 0 as its anchor against the causal decode of block
    1's queries over the whole context (both on the GPU, both to the bar)."""
    Lb, Hq, Hkv, D = 500, 32, 8, 128
    q, k0, v0, k1, v1 = make(1, Lb, Hq, Hkv, D, Lb, seed=3)
    scale = 1.0 / np.sqrt(D)
    O, lse = binding.prefill_anchor(dev(q), dev(k0), dev(v0), dev(k1), dev(v1), scale=scale)
    kc = np.concatenate([k0[None], k1], axis=2)  # [1][Hkv][2Lb][D]
    vc = np.concatenate([v0[None], v1], axis=2)
    Og, lg = binding.decode(dev(q), dev(kc), dev(vc), scale=scale, causal=True)
    torch.cuda.synchronize()
    Or, lr = oracle.attend(q, kc, vc, [2 * Lb], scale, causal=True)
    check_rows(O.cpu().numpy(), lse.cpu().numpy(), Or, lr, what="block 1 with anchor")
    check_rows(Og.cpu().numpy(), lg.cpu().numpy(), Or, lr, what="global causal decode")


def test_anchor_blocks_bench_shape_sampled():
    """Two 8192-token blocks behind an 8192-token anchor, 32 query / 8 KV
    heads, d = 128: the first, middle and last query tokens of each block on
    every head against the oracle."""
    N, Lb, Hq, Hkv, D, A = 2, 8192, 32, 8, 128, 8192
    q, ka, va, kb, vb = make(N, Lb, Hq, Hkv, D, A, seed=41)
    scale = 1.0 / np.sqrt(D)
    O, lse = binding.prefill_anchor(dev(q), dev(ka), dev(va), dev(kb), dev(vb), scale=scale)
    torch.cuda.synchronize()
    rows = [(b, i, h) for b in range(N) for i in (0, 1, Lb // 2, Lb - 1) for h in range(Hq)]
    Or, lr = oracle.attend_anchor_blocks(q, ka, va, kb, vb, scale, rows=rows)
    check_rows(O.cpu().numpy(), lse.cpu().numpy(), Or, lr, rows=rows, what="anchor bench shape")


def test_anchor_too_small_workspace_is_refused():
    """A workspace one byte short: ATTN_ERR_WORKSPACE and untouched outputs."""
    import ctypes
    lib = binding.load_library()
    q, ka, va, kb, vb = make(2, 100, 8, 2, 128, 300, seed=3)
    t = [dev(x) for x in (q, ka, va, kb, vb)]
    d = binding.anchor_desc(t[0], t[1], t[3], 1.0 / np.sqrt(128))
    n = ctypes.c_size_t(0)
    assert lib.attn_anchor_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == 0 and n.value > 0
    ws = torch.empty(n.value, dtype=torch.uint8, device="cuda")
    O = torch.full((2, 100, 8, 128), 7.0, device="cuda")
    lse = torch.full((2, 100, 8), 7.0, device="cuda")
    st = lib.attn_prefill_anchor(ctypes.byref(d), *[x.data_ptr() for x in t], O.data_ptr(),
                                 lse.data_ptr(), ws.data_ptr(), n.value - 1,
                                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert binding.STATUS[st] == "ATTN_ERR_WORKSPACE"
    assert (O == 7.0).all() and (lse == 7.0).all()
