"""The fp64 oracle against its pins (CPU only)."""
import math

import numpy as np
import pytest

import oracle
import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((2, 3, 4, 5)); k = rng.standard_normal((2, 2, 40, 5))
    v = rng.standard_normal((2, 2, 40, 5))
    O, lse = oracle.attend(q, k, v, [40, 13], 0.5, True)
    rows = [(1, 2, 3), (0, 0, 0), (1, 0, 2)]
    Os, ls = oracle.attend(q, k, v, [40, 13], 0.5, True, rows=rows)
    for (b, i, h) in rows:
        # a different row set changes only BLAS blocking, i.e. the last bits
        assert np.allclose(Os[b, i, h], O[b, i, h], rtol=1e-14, atol=1e-15)
        assert abs(ls[b, i, h] - lse[b, i, h]) <= 1e-14 * abs(lse[b, i, h])
    assert np.isnan(ls[0, 1, 1])


def test_slab_streaming_is_exact_rewrite():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 2, 4)); k = rng.standard_normal((1, 1, 101, 4))
    v = rng.standard_normal((1, 1, 101, 4))
    O, lse = oracle.attend(q, k, v, [101], 0.5)
    O7, l7 = oracle.attend(q, k, v, [101], 0.5, slab=7)
    assert np.allclose(O7, O, rtol=1e-13, atol=1e-14) and np.allclose(l7, lse, rtol=1e-14)


def test_energy_only_mode():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 2, 4)); k = rng.standard_normal((1, 1, 20, 4))
    v = rng.standard_normal((1, 1, 20, 4))
    O, lse = oracle.attend(q, k, v, [20], 0.5)
    none, lse_e = oracle.attend(q, k, None, [20], 0.5)
    assert none is None and np.array_equal(lse_e, lse)


def test_bf16_bits_are_widened_exactly():
    # 0x3FC0 = 1.5, 0xC040 = -3.0, 0x4049 = 3.140625 in bfloat16
    q = np.array([[[[0x3FC0, 0x0000]]]], dtype=np.uint16)
    k = np.array([[[[0xC040, 0x4049]]]], dtype=np.uint16)
    v = np.array([[[[0x4049, 0x3FC0]]]], dtype=np.uint16)
    O, lse = oracle.attend(q, k, v, [1], 1.0)
    assert lse[0, 0, 0] == -4.5
    assert np.array_equal(O[0, 0, 0], [3.140625, 1.5])


def test_needle_row_is_near_its_closed_form():
    """One key whose logit exceeds all others by ~25: lse - s_n and |O - v_n|
    are bounded by the weight left to the other keys."""
    rng = np.random.default_rng(3)
    L, D, sc = 4096, 16, 0.25
    q = rng.standard_normal(D); k = rng.standard_normal((L, D)); v = rng.standard_normal((L, D))
    n = 1234
    k[n] = (30.0 / (sc * np.linalg.norm(q))) * q / np.linalg.norm(q)
    O, lse = oracle.attend(q[None, None, None], k[None, None], v[None, None], [L], sc)
    s = sc * (k @ q)
    others = np.delete(s, n)
    upper = math.log1p(float(np.exp(others - s[n]).sum()))
    assert 0.0 <= lse[0, 0, 0] - s[n] <= upper * (1 + 1e-9) + 1e-15
    w_rest = 1.0 - math.exp(s[n] - lse[0, 0, 0])
    assert np.abs(O[0, 0, 0] - v[n]).max() <= 2 * w_rest * np.abs(v).max() + 1e-12


def test_finalised_share_results_merge_as_records():
    """The reading behind merging per-share results (a sequence-sharded
    decode): a finalised result (O, lse) over some keys is the record
    (m = lse, l = 1, o = O), so merging the shares' results with the merge
    rule, in any order, gives attention over all the keys; a share with no
    visible key (lse = -inf) is the identity."""
    import random
    rng = np.random.default_rng(37)
    rnd = random.Random(37)
    for case in range(12):
        L = int(rng.integers(1, 90))
        D = int(rng.integers(1, 9))
        q = rng.standard_normal((1, 1, 1, D))
        k = rng.standard_normal((1, 1, L, D)) * 2.0
        v = rng.standard_normal((1, 1, L, D))
        O, lse = oracle.attend(q, k, v, [L], 0.7)
        cuts = sorted({0, L, *rng.integers(0, L + 1, size=int(rng.integers(0, 5))).tolist()})
        recs = []
        for c0, c1 in zip(cuts[:-1], cuts[1:]):
            Os, ls = oracle.attend(q, k[:, :, c0:c1], v[:, :, c0:c1], [c1 - c0], 0.7)
            recs.append((float(ls[0, 0, 0]), 1.0, Os[0, 0, 0]))
        recs.append((-math.inf, 0.0, np.zeros(D)))  # an empty share
        rnd.shuffle(recs)
        acc = recs[0]
        for r in recs[1:]:
            acc = oracle.merge(acc, r)
        Om, lm = oracle.finalize(acc)
        assert np.allclose(Om, O[0, 0, 0], rtol=1e-12, atol=1e-13), case
        assert abs(lm - lse[0, 0, 0]) <= 1e-12 * max(1.0, abs(lse[0, 0, 0])), case
