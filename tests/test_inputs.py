"""Seeded workload generator: rounding, reproducibility and planted structure."""
import math

import numpy as np
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
