"""attn_decode_static (no workspace, no allocation) against attn_decode.

The static entry point runs the same kernels with the partial records in
the library's device array instead of a caller workspace, so on the same
inputs its O and lse must equal attn_decode's bit for bit (and so meet the
parity bar against them).  Two calls in a row, the second on a smaller
input, check that the array's leftovers from one call never leak into the
next; a query-block shape takes the matrix-core kernel; a call that needs
more record space than the array holds is refused before any launch, with
its outputs untouched.
"""
import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import LSE_RTOL, O_TOL, say, workload_tensors
from long_context_exact_split_amd import binding, inputs

pytestmark = pytest.mark.gpu


def _both(w):
    q, k, v, lens = workload_tensors(w)
    O1, l1 = binding.decode(q, k, v, lens, scale=w.scale, causal=w.causal, chunk_len=w.chunk_len)
    O2, l2 = binding.decode_static(q, k, v, lens, scale=w.scale, causal=w.causal,
                                   chunk_len=w.chunk_len)
    torch.cuda.synchronize()
    return (x.cpu().numpy() for x in (O1, l1, O2, l2))


def _check(w, what):
    O1, l1, O2, l2 = _both(w)
    say(f"{what}: max|dO|={np.abs(O1 - O2).max():.2e}")
    fin = np.isfinite(l1)
    assert (l2[~fin] == l1[~fin]).all()
    assert np.abs(O1 - O2).max() <= O_TOL
    assert (np.abs(l1[fin] - l2[fin]) <= LSE_RTOL * np.maximum(1.0, np.abs(l1[fin]))).all()
    assert np.array_equal(O1, O2) and np.array_equal(l1, l2), "not bitwise equal"


def test_static_matches_workspace_entry_point_twice_in_a_row():
    big = inputs.make_decode("noalloc_big", 41, B=3, q_len=1, Hq=32, Hkv=8, D=128, L_max=50000,
                             kv_lens=[50000, 17, 31999], nan_pad=True)
    small = inputs.make_decode("noalloc_small", 42, B=1, q_len=1, Hq=8, Hkv=2, D=128, L_max=3000)
    _check(big, "static vs workspace, 3 x 50000 tokens")
    _check(small, "static vs workspace, 1 x 3000 tokens (second call, smaller)")


def test_static_query_blocks_on_the_matrix_cores():
    w = inputs.make_decode("noalloc_qb", 43, B=2, q_len=4, Hq=64, Hkv=8, D=128, L_max=20000,
                           kv_lens=[20000, 7000], causal=True, nan_pad=True)
    d = binding.make_desc(batch=2, q_len=4, num_q_heads=64, num_kv_heads=8, head_dim=128,
                          max_kv_len=20000, causal=True)
    assert binding.plan(d)["kernel"] == 1
    _check(w, "static vs workspace, 32-row query blocks")


def test_static_refuses_calls_beyond_the_array():
    # 64-token chunks of a 100000-token cache: ~26 MB of records > 16 MiB
    B, Hq, Hkv, D, L = 1, 32, 8, 128, 100000
    d = binding.make_desc(batch=B, q_len=1, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                          max_kv_len=L, chunk_len=64)
    assert binding.workspace_bytes(d) > 16 << 20
    q = torch.zeros((B, 1, Hq, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, L, D), dtype=torch.bfloat16, device="cuda")
    o = torch.full((B, 1, Hq, D), 7.0, device="cuda")
    lse = torch.full((B, 1, Hq), 7.0, device="cuda")
    st = binding.load_library().attn_decode_static(ctypes.byref(d), q.data_ptr(), k.data_ptr(),
                                                   k.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert binding.STATUS[st] == "ATTN_ERR_SCRATCH"
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
