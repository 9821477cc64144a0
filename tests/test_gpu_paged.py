"""Paged KV caches on the GPU (through the C ABI) against the fp64 oracle.

The pools are built by the input generator (seeded random physical page
order, NaN in every page slot no sequence uses, -1 in unused table entries);
the oracle resolves the same pools and block table itself (oracle.gather) and
applies the plain definition.  Paging only changes where rows are read, so
the paged call must also reproduce the dense call on the same logical cache
bit for bit (same plan, same arithmetic).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import check_rows, dev, say, workload_tensors
from long_context_exact_split_amd import binding, inputs

pytestmark = pytest.mark.gpu


def paged_tensors(w, pc):
    B, Hkv, D = w.B, w.Hkv, w.D
    P = pc.page_size
    shape = (pc.num_pages, Hkv, P, D) if pc.layout == "head_major" else (pc.num_pages, P, Hkv, D)
    kp = dev(pc.k_pool.reshape(shape))
    vp = dev(pc.v_pool.reshape(shape))
    table = torch.from_numpy(pc.block_table).cuda()
    cache = binding.PagedCache(kp, vp, table, layout=pc.layout, max_kv_len=w.L_max)
    lens = torch.from_numpy(w.kv_lens.astype(np.int32)).cuda()
    return cache, lens


def oracle_paged(w, pc, rows=None, energy=False):
    return oracle.attend_paged(w.q, pc.k_pool, None if energy else pc.v_pool, pc.block_table,
                               w.kv_lens, w.scale, page_size=pc.page_size,
                               page_stride=pc.page_stride, head_stride=pc.head_stride,
                               token_stride=pc.token_stride, num_kv_heads=w.Hkv, L_max=w.L_max,
                               causal=w.causal, rows=rows)


PAGED = [
    # B, q_len, Hq, Hkv, D, L, dtype, causal, lens, P, layout, shared prefix tokens, spare pages
    (1, 1, 32, 8, 128, 5000, "bf16", False, None, 16, "head_major", 0, 3),
    (3, 1, 32, 8, 128, 3000, "bf16", False, [3000, 0, 1717], 16, "token_major", 0, 5),
    (2, 1, 8, 8, 64, 2049, "bf16", False, [2049, 600], 1, "head_major", 0, 0),
    (4, 1, 10, 2, 128, 1234, "f32", False, "uniform:1:1234", 32, "token_major", 0, 2),
    (2, 1, 4, 4, 64, 999, "f32", False, [999, 64], 8, "head_major", 0, 1),
    (3, 1, 16, 4, 128, 4096, "bf16", False, [4096, 3000, 2500], 64, "head_major", 2048, 4),
    (2, 4, 64, 8, 128, 4500, "bf16", True, [4500, 4096], 16, "head_major", 0, 1),
    (2, 8, 64, 8, 128, 3000, "bf16", True, [3000, 1000], 16, "token_major", 0, 1),
    (1, 1, 256, 1, 128, 3000, "bf16", False, None, 16, "head_major", 0, 0),
    (1, 2, 8, 1, 64, 1000, "bf16", True, None, 8, "token_major", 0, 0),
    (2, 4, 16, 2, 128, 1500, "bf16", True, [1500, 1100], 1024, "head_major", 1024, 0),
    (2, 6, 16, 1, 128, 2000, "bf16", True, [2000, 900], 32, "token_major", 512, 2),
    # causal query blocks over several row blocks of 256 (each sees only its keys)
    (1, 96, 8, 2, 128, 700, "bf16", True, None, 16, "head_major", 0, 1),
    (2, 130, 16, 4, 64, 900, "bf16", True, [900, 300], 32, "token_major", 0, 2),
]


def _id(c):
    return (f"B{c[0]}_ql{c[1]}_Hq{c[2]}_Hkv{c[3]}_D{c[4]}_L{c[5]}_{c[6]}_P{c[9]}_{c[10]}"
            + ("_causal" if c[7] else "") + (f"_share{c[11]}" if c[11] else ""))


@pytest.mark.parametrize("case", PAGED, ids=[_id(c) for c in PAGED])
def test_paged_small_shapes(case):
    B, q_len, Hq, Hkv, D, L, dt, causal, lens, P, layout, share, spare = case
    say(f"paged case {_id(case)}")
    w = inputs.make_decode("paged", 500 + L, B=B, q_len=q_len, Hq=Hq, Hkv=Hkv, D=D, L_max=L,
                           kv_lens=lens, dtype=dt, causal=causal, nan_pad=True)
    pc = inputs.page_cache(w, P, layout=layout, seed=L, spare_pages=spare,
                           share_prefix_tokens=share)
    cache, lens_t = paged_tensors(w, pc)
    q = dev(w.q)
    O, lse = binding.decode_paged(q, cache, lens_t, scale=w.scale, causal=causal)
    lse_e = binding.decode_energy_paged(q, cache, lens_t, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    Or, lr = oracle_paged(w, pc)
    check_rows(O.cpu().numpy(), lse.cpu().numpy(), Or, lr, what=f"paged {_id(case)}")
    check_rows(None, lse_e.cpu().numpy(), None, lr, what=f"paged energy {_id(case)}")
    # The dense call on the same logical cache gives the same bits.
    qd, kd, vd, ld = workload_tensors(w)
    Od, lsed = binding.decode(qd, kd, vd, ld, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(O, Od) and torch.equal(lse, lsed), "paged and dense results differ"


def test_paged_long_context_1m_sampled():
    """1,048,576-token GQA decode in 16-token head-major pages (65,536 pages in
    a random order): every row checked against the oracle, the needle heads
    among them."""
    w = inputs.long_context_gqa(L=1 << 20, seed=31)
    pc = inputs.page_cache(w, 16, layout="head_major", seed=7)
    say(f"paged 1M: {pc.num_pages} pages")
    cache, lens_t = paged_tensors(w, pc)
    q = dev(w.q)
    O, lse = binding.decode_paged(q, cache, lens_t, scale=w.scale)
    torch.cuda.synchronize()
    rows = [(0, 0, h) for h in range(w.Hq)]
    Or, lr = oracle_paged(w, pc, rows=rows)
    check_rows(O.cpu().numpy(), lse.cpu().numpy(), Or, lr, rows=rows, what="paged 1M GQA")
    # The needle key is rounded to bf16 after being scaled to logit 30, which
    # moves that logit by up to ~2^-8 of itself; it still dominates its row.
    for (_, kvh, _) in w.notes["needles"]:
        assert abs(float(lse[0, 0, kvh * w.G]) - 30.0) < 0.15


def test_paged_llama31_70b_ragged_sampled():
    """The 70B-shaped ragged batch (4 causal query tokens, MFMA path) in
    16-token token-major pages; two sequences' rows against the oracle."""
    w = inputs.llama31_70b_ragged(seed=5)
    pc = inputs.page_cache(w, 16, layout="token_major", seed=9, spare_pages=64)
    cache, lens_t = paged_tensors(w, pc)
    q = dev(w.q)
    O, lse = binding.decode_paged(q, cache, lens_t, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    b_short, b_long = int(np.argmin(w.kv_lens)), int(np.argmax(w.kv_lens))
    rows = [(b, i, h) for b in (b_short, b_long) for i in range(w.q_len) for h in range(w.Hq)]
    Or, lr = oracle_paged(w, pc, rows=rows)
    check_rows(O.cpu().numpy(), lse.cpu().numpy(), Or, lr, rows=rows, what="paged 70B ragged")
