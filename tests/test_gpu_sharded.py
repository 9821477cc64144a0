"""Sequence-sharded decoding on one GPU: the cache of every sequence is cut
into token shares (one per device in a sharded deployment), each share is
decoded by attn_decode on its own copy, and attn_merge_results combines the
per-share (O, lse) pairs (the exchange step: Star Attention article, phase 2;
Tree Attention article, "an energy view of attention").  The merged result
is compared with the fp64 oracle over the whole cache, element by element,
and with the one-call decode of the whole cache."""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import check_rows, dev, say, workload_tensors
from long_context_exact_split_amd import binding, inputs

pytestmark = pytest.mark.gpu


def decode_shares(q, k, v, kv_lens, cuts, scale):
    """(O_p, lse_p) of every share [cuts[j], cuts[j+1]) of the token axis,
    stacked on a new leading axis.  A sequence holding L_b tokens sees
    clamp(L_b - c0, 0, c1 - c0) of a share's tokens."""
    O_parts, lse_parts = [], []
    for c0, c1 in zip(cuts[:-1], cuts[1:]):
        ks = k[:, :, c0:c1].contiguous()
        vs = v[:, :, c0:c1].contiguous()
        lens = torch.clamp(kv_lens - c0, 0, c1 - c0).to(torch.int32).contiguous()
        O, lse = binding.decode(q, ks, vs, lens, scale=scale)
        O_parts.append(O)
        lse_parts.append(lse)
        del ks, vs
    return torch.stack(O_parts), torch.stack(lse_parts)


# B, Hq, Hkv, D, L_max, lens, cuts, dtype
CASES = [
    (2, 8, 2, 128, 3000, [3000, 1111], [0, 1000, 2200, 3000], "bf16"),    # empty shares
    (3, 16, 16, 64, 4096, [4096, 4000, 17], [0, 512, 1024, 1536, 2048, 2560, 3072, 3584, 4096],
     "bf16"),                                                              # G = 1, eight shares
    (1, 32, 8, 128, 2048, [2048], [0, 2048], "bf16"),                      # one share
    (1, 4, 1, 128, 70 * 64, [70 * 64 - 5], list(range(0, 70 * 64 + 1, 64)), "bf16"),  # 70 shares
    (1, 1, 1, 64, 4096, [4096], [0, 512, 1024, 1536, 2048, 2560, 3072, 3584, 4096], "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_Hq{c[1]}_Hkv{c[2]}_D{c[3]}_n{len(c[6]) - 1}_{c[7]}"
                                             for c in CASES])
def test_sharded_decode_matches_oracle(case):
    B, Hq, Hkv, D, L, lens, cuts, dtype = case
    w = inputs.make_decode("sharded", 41 + len(cuts), B=B, q_len=1, Hq=Hq, Hkv=Hkv, D=D,
                           L_max=L, kv_lens=lens, dtype=dtype, nan_pad=True)
    q, k, v, _ = workload_tensors(w)
    kv_lens = torch.from_numpy(w.kv_lens.astype(np.int32)).cuda()
    O_parts, lse_parts = decode_shares(q, k, v, kv_lens, cuts, w.scale)
    O, lse = binding.merge_results(O_parts, lse_parts)
    O1, lse1 = binding.decode(q, k, v, kv_lens, scale=w.scale)
    torch.cuda.synchronize()
    Or, lr = oracle.attend(w.q, w.k, w.v, w.kv_lens, w.scale, False)
    check_rows(O.cpu().numpy(), lse.cpu().numpy(), Or, lr, what=f"sharded {case[:5]}")
    # the same rows as the one-call decode, up to the order of the merge
    assert torch.allclose(O, O1, atol=2e-5, rtol=0)
    assert torch.allclose(lse, lse1, atol=2e-5, rtol=1e-6)
    # energies only: each share's lse from K alone, reduced to the whole cache's
    e_parts = []
    for c0, c1 in zip(cuts[:-1], cuts[1:]):
        lens = torch.clamp(kv_lens - c0, 0, c1 - c0).to(torch.int32).contiguous()
        e_parts.append(binding.decode_energy(q, k[:, :, c0:c1].contiguous(), lens, scale=w.scale))
    lse_e = binding.merge_energies(torch.stack(e_parts))
    torch.cuda.synchronize()
    check_rows(None, lse_e.cpu().numpy(), None, lr, what=f"sharded energy {case[:5]}")
    assert torch.allclose(lse_e, lse, atol=2e-5, rtol=1e-6)


def test_merge_results_edge_rows():
    """Parts that saw no key (lse = -inf, O = NaN) add nothing; a row whose
    every part is empty gives O = 0 and lse = -inf; parts whose lse differ by
    ~160 merge without overflow.  Expected values: the oracle's merge of the
    records (m = lse_p, l = 1, o = O_p)."""
    rng = np.random.default_rng(5)
    n, rows, D = 11, 37, 128
    lse_p = rng.normal(0.0, 40.0, size=(n, rows)).astype(np.float32)
    O_p = rng.standard_normal((n, rows, D)).astype(np.float32)
    empty = rng.random((n, rows)) < 0.3
    empty[:, 3] = True            # a row that sees no key at all
    empty[:, 4] = False
    lse_p[0, 4], lse_p[1, 4] = 80.0, -80.0
    lse_p[empty] = -np.inf
    O_p[empty] = np.nan
    O, lse = binding.merge_results(dev(O_p), dev(lse_p))
    torch.cuda.synchronize()
    O, lse = O.cpu().numpy(), lse.cpu().numpy()
    assert not np.isnan(O).any() and not np.isnan(lse).any()
    Or = np.zeros((rows, D))
    lr = np.zeros(rows)
    for r in range(rows):
        rec = (-math.inf, 0.0, np.zeros(D))
        for p in range(n):
            if not empty[p, r]:
                rec = oracle.merge(rec, (float(lse_p[p, r]), 1.0, O_p[p, r].astype(np.float64)))
        Or[r], lr[r] = oracle.finalize(rec)
    assert lse[3] == -np.inf and (O[3] == 0).all()
    check_rows(O[:, None, None], lse[:, None, None], Or[:, None, None], lr[:, None, None],
               what="merge_results edge rows")


def test_merge_results_wide_rows_and_output_checks():
    """Rows given as [n, B, Hq, D] with 130 parts (more than one per lane of a
    wave); caller-supplied outputs of the wrong dtype are refused before the
    call."""
    rng = np.random.default_rng(9)
    n, B, Hq, D = 130, 2, 3, 64
    lse_p = rng.normal(5.0, 3.0, size=(n, B, Hq)).astype(np.float32)
    O_p = rng.standard_normal((n, B, Hq, D)).astype(np.float32)
    O, lse = binding.merge_results(dev(O_p), dev(lse_p))
    torch.cuda.synchronize()
    M = lse_p.astype(np.float64).max(axis=0)
    wgt = np.exp(lse_p - M)
    Or = (wgt[..., None] * O_p).sum(axis=0) / wgt.sum(axis=0)[..., None]
    lr = M + np.log(wgt.sum(axis=0))
    check_rows(O.cpu().numpy()[:, None], lse.cpu().numpy()[:, None], Or[:, None], lr[:, None],
               what="merge_results 130 parts")
    with pytest.raises(ValueError):
        binding.merge_results(dev(O_p), dev(lse_p), out=torch.empty((B, Hq, D), device="cuda",
                                                                    dtype=torch.bfloat16))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_long_context_5m_in_eight_shares():
    """The 5.12M-token cache as eight devices would hold it (640,000 tokens
    each): eight share decodes at their real shape, merged, against the oracle
    on the needle rows (each needle lies in one share, so the merge must keep
    the dominant share's statistics) and against the one-call decode."""
    w = inputs.long_context_gqa(L=5_120_000, seed=3)
    say("generated 5.12M-token cache")
    q, k, v, lens = workload_tensors(w)
    kv_lens = torch.full((1,), w.L_max, dtype=torch.int32, device="cuda")
    cuts = list(range(0, 5_120_001, 640_000))
    O_parts, lse_parts = decode_shares(q, k, v, kv_lens, cuts, w.scale)
    O, lse = binding.merge_results(O_parts, lse_parts)
    O1, lse1 = binding.decode(q, k, v, lens, scale=w.scale)
    torch.cuda.synchronize()
    say("eight shares decoded and merged")
    assert torch.allclose(O, O1, atol=2e-5, rtol=0)
    assert torch.allclose(lse, lse1, atol=1e-4, rtol=1e-6)
    O, lse = O.cpu().numpy(), lse.cpu().numpy()
    del q, k, v, O_parts, lse_parts
    torch.cuda.empty_cache()
    rows = [(0, 0, w.G * kvh) for (_, kvh, _) in w.notes["needles"]] + [(0, 0, 1), (0, 0, 29)]
    from test_gpu_parity import oracle_decode_parallel
    Or, lr = oracle_decode_parallel(w, rows)
    check_rows(O, lse, Or, lr, rows=rows, what="5.12M in eight shares")
