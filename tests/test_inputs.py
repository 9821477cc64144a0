"""Seeded workload generator: rounding, reproducibility and planted structure."""
import math

import numpy as np
import pytest
import torch

from long_context_exact_split_amd import inputs


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.4e38, 1e-40,
                                  1.00390625, 1.01171875], np.float32)])  # ties
    ours = inputs.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = inputs.bf16_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    assert inputs.f32_to_bf16(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_seeds_reproducible_and_distinct():
    a = inputs.make_decode("t", 5, B=2, q_len=1, Hq=4, Hkv=2, D=16, L_max=300)
    b = inputs.make_decode("t", 5, B=2, q_len=1, Hq=4, Hkv=2, D=16, L_max=300)
    c = inputs.make_decode("t", 6, B=2, q_len=1, Hq=4, Hkv=2, D=16, L_max=300)
    for f in ("q", "k", "v"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
        assert not np.array_equal(getattr(a, f), getattr(c, f))


def test_slabs_independent_of_thread_schedule():
    # two slabs per sequence; the content is fixed by the seed, not the thread order
    a = inputs.make_decode("t", 9, B=2, q_len=1, Hq=2, Hkv=1, D=8, L_max=inputs.SLAB_TOKENS + 17)
    b = inputs.make_decode("t", 9, B=2, q_len=1, Hq=2, Hkv=1, D=8, L_max=inputs.SLAB_TOKENS + 17)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    kf = a.values("k")
    assert abs(float(kf.mean())) < 0.01 and abs(float(kf.std()) - 1.0) < 0.01


def test_single_query_fp32_shape():
    w = inputs.single_query_fp32()
    assert w.dtype == "f32" and w.q.dtype == np.float32
    assert w.q.shape == (1, 1, 1, 64) and w.k.shape == (1, 1, 4096, 64)
    assert w.chunk_len == 512 and w.scale == 1.0 / 8.0


def test_needle_logit_dominates():
    w = inputs.long_context_gqa(L=20000, seed=3)
    assert len(w.notes["needles"]) == 8
    qf = w.values("q").astype(np.float64)
    for (b, kvh, n) in w.notes["needles"]:
        kf = inputs.bf16_to_f32(w.k[b, kvh, n]).astype(np.float64)
        logit = w.scale * float(qf[b, 0, w.G * kvh] @ kf)
        assert abs(logit - 30.0) < 0.2, logit
    lit = inputs.long_context_gqa(L=20000, seed=3, literal_c=6.0)
    (b, kvh, n) = lit.notes["needles"][0]
    kf = inputs.bf16_to_f32(lit.k[b, kvh, n]).astype(np.float64)
    assert abs(np.linalg.norm(kf) - 6.0) < 0.05


def test_ragged_heavy_tail_and_nan_padding():
    w = inputs.llama31_70b_ragged(seed=5, L_max=4096, L_lo=256, B=4)
    assert w.kv_lens.dtype == np.int32
    assert ((w.kv_lens >= 256) & (w.kv_lens <= 4096)).all()
    for b in range(w.B):
        L = int(w.kv_lens[b])
        assert (w.k[b, :, L:] == 0x7FC0).all() and (w.v[b, :, L:] == 0x7FC0).all()
        assert not np.isnan(w.values("k")[b, :, :L]).any()
    frac = w.notes["heavy_rows"] / (w.Hkv * w.kv_lens.sum())
    assert 0.004 < frac < 0.02
    kf = w.values("k")[:, :, :256]
    big = (np.abs(kf).max(axis=-1) > 12).mean()
    assert big > 0.002  # x8 rows are visible in the data


def test_lengths_drawn_inclusive_uniform():
    w = inputs.make_decode("t", 1, B=64, q_len=1, Hq=1, Hkv=1, D=4, L_max=16,
                           kv_lens="uniform:14:16")
    assert set(np.unique(w.kv_lens).tolist()) == {14, 15, 16}


def test_bifurcated_shapes():
    w = inputs.bifurcated_prefix(S=4, Lp=300, Ls=40)
    assert w.q.shape == (4, 32, 128) and w.kp.shape == (8, 300, 128)
    assert w.ks.shape == (4, 8, 40, 128) and w.scale == 1 / math.sqrt(128)


@pytest.mark.parametrize("layout", ["head_major", "token_major"])
def test_page_cache_resolves_to_the_dense_cache(layout):
    import oracle
    w = inputs.make_decode("t", 12, B=3, q_len=1, Hq=4, Hkv=2, D=8, L_max=70,
                           kv_lens=[70, 0, 33])
    pc = inputs.page_cache(w, 16, layout=layout, seed=1, spare_pages=5)
    assert pc.num_pages == 5 + 3 + 5 and pc.pages_per_seq == 5
    t = pc.block_table
    assert (t[1] == -1).all() and (t[2, 3:] == -1).all() and (t[0] >= 0).all()
    used = t[t >= 0]
    assert len(set(used.tolist())) == used.size  # no page stored twice
    dense = oracle.gather(pc.k_pool, t, w.kv_lens, pc.page_size, pc.page_stride, pc.head_stride,
                          pc.token_stride, w.Hkv, w.D, w.L_max)
    for b, L in enumerate(w.kv_lens):
        assert np.array_equal(dense[b, :, :L], w.k[b, :, :L])
    spare = np.setdiff1d(np.arange(pc.num_pages), used)
    pool = pc.k_pool.reshape(pc.num_pages, -1)
    assert (pool[spare] == inputs.BF16_NAN).all()


def test_page_cache_shares_prefix_pages():
    import oracle
    w = inputs.make_decode("t", 13, B=3, q_len=1, Hq=2, Hkv=1, D=8, L_max=64, kv_lens=[64, 40, 50])
    pc = inputs.page_cache(w, 8, share_prefix_tokens=20, seed=2)
    assert pc.shared_pages == 2
    t = pc.block_table
    assert (t[1, :2] == t[0, :2]).all() and (t[2, :2] == t[0, :2]).all()
    assert np.array_equal(w.k[1, :, :20], w.k[0, :, :20])  # the logical caches now share tokens
    dense = oracle.gather(pc.v_pool, t, w.kv_lens, 8, pc.page_stride, pc.head_stride,
                          pc.token_stride, 1, 8, 64)
    for b, L in enumerate(w.kv_lens):
        assert np.array_equal(dense[b, :, :L], w.v[b, :, :L])
