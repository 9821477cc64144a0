"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them: a dropped scale, a wrong GQA index, an off-by-one
causal window, K and V swapped, a log2 logsumexp, a missing normalisation,
an unshifted exponential, a merge that forgets to rescale, an energy that
drops its zeta term, paged-cache lookups with swapped strides, an ignored
block table or quotient and remainder exchanged, row energies that ignore
the causal window or the GQA grouping, and an anchor placed after the block
or a block attended without its causal mask.  None of these variants is used anywhere else."""
import math
import types

import numpy as np
import pytest

import oracle
import oracle_pins as pins


def _row(q, k, v, scale, mistake):
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    n = k.shape[0]
    if n == 0:
        return np.zeros(v.shape[1]), -math.inf
    if mistake == "kv_swapped":
        k, v = v, k
    s = (1.0 if mistake == "no_scale" else scale) * (k @ q)
    if mistake == "sign":
        s = -s
    if mistake == "no_max_shift":
        with np.errstate(over="ignore", invalid="ignore"):
            e = np.exp(s)
            return (e @ v) / e.sum(), math.log(e.sum()) if np.isfinite(e.sum()) else math.nan
    M = s.max()
    e = np.exp(s - M)
    lse = M + math.log(e.sum())
    if mistake == "lse_log2":
        lse = lse / math.log(2.0)
    if mistake == "lse_drops_max":
        lse = math.log(e.sum())
    if mistake == "unnormalised":
        return e @ v, lse
    return (e / e.sum()) @ v, lse


def _attend_factory(mistake):
    def attend(q, k, v, kv_lens, scale, causal=False, rows=None, slab=0):
        B, q_len, Hq, D = q.shape
        Hkv = k.shape[1]
        G = Hq // Hkv
        O = np.zeros((B, q_len, Hq, v.shape[-1])) if v is not None else None
        lse = np.zeros((B, q_len, Hq))
        for b in range(B):
            for i in range(q_len):
                Lb = int(kv_lens[b])
                if causal and mistake != "causal_ignored":
                    n = Lb - q_len + i + (0 if mistake == "causal_off_by_one" else 1)
                else:
                    n = Lb
                n = max(0, min(Lb, n))
                for h in range(Hq):
                    kvh = h % Hkv if mistake == "gqa_modulo" else h // G
                    vv = v[b, kvh, :n] if v is not None else k[b, kvh, :n]
                    o, l = _row(q[b, i, h], k[b, kvh, :n], vv, scale, mistake)
                    if O is not None:
                        O[b, i, h] = o
                    lse[b, i, h] = l
        return O, lse
    return attend


def _merge_factory(mistake):
    def merge(a, b):
        ma, la, oa = a
        mb, lb, ob = b
        m = max(ma, mb)
        if m == -math.inf:
            return (-math.inf, 0.0, np.zeros_like(oa))
        wa = math.exp(ma - m) if ma != -math.inf else 0.0
        wb = math.exp(mb - m) if mb != -math.inf else 0.0
        if mistake == "merge_no_rescale_o":
            return (m, la * wa + lb * wb, oa + ob)
        if mistake == "merge_inverted_weight":
            wa = math.exp(m - ma) if ma != -math.inf else 0.0
            wb = math.exp(m - mb) if mb != -math.inf else 0.0
        return (m, la * wa + lb * wb, oa * wa + ob * wb)
    return merge


def _energy_factory(mistake):
    def energy(q, k, v, scale, zeta=None):
        if mistake == "energy_no_zeta":
            zeta = None
        if mistake == "energy_scaled_zeta" and zeta is not None:
            zeta = scale * np.asarray(zeta)
        return oracle.energy(q, k, v, scale, zeta)
    return energy


def _bif_factory(attend):
    def attend_bifurcated(q, kp, vp, ks, vs, scale, samples=None):
        S, Hq, D = q.shape
        O = np.zeros((S, Hq, D)); lse = np.zeros((S, Hq))
        for s in range(S):
            kc = np.concatenate([kp, ks[s]], axis=1)[None]
            vc = np.concatenate([vp, vs[s]], axis=1)[None]
            o, l = attend(q[s][None, None], kc, vc, [kc.shape[2]], scale)
            O[s], lse[s] = o[0, 0], l[0, 0]
        return O, lse
    return attend_bifurcated


def _gather_factory(mistake):
    def gather(pool, table, kv_lens, P, ps, hs, ts, Hkv, D, L_max):
        pool = np.asarray(pool).reshape(-1)
        if mistake == "page_strides_swapped":
            hs, ts = ts, hs
        B = len(kv_lens)
        out = np.full((B, Hkv, L_max, D), np.nan)
        for b in range(B):
            for t in range(int(kv_lens[b])):
                j, slot = t // P, t % P
                if mistake == "page_quotient_remainder_swapped":
                    j, slot = slot % np.shape(table)[1], j % P
                page = b * np.shape(table)[1] + j if mistake == "page_ignores_table" else table[b][j]
                for h in range(Hkv):
                    r = page * ps + h * hs + slot * ts
                    out[b, h, t] = pool[r:r + D]
        return out
    return gather


def _attend_paged_factory(attend, gather):
    def attend_paged(q, k_pool, v_pool, table, kv_lens, scale, *, page_size, page_stride,
                     head_stride, token_stride, num_kv_heads, L_max, causal=False, rows=None):
        geo = (page_size, page_stride, head_stride, token_stride, num_kv_heads, q.shape[-1], L_max)
        k = gather(k_pool, table, kv_lens, *geo)
        v = None if v_pool is None else gather(v_pool, table, kv_lens, *geo)
        return attend(q, k, v, kv_lens, scale, causal)
    return attend_paged


def _energy_rows_factory(energy, mistake):
    def energy_rows(q, k, v, kv_lens, scale, zeta, causal=False, rows=None):
        B, q_len, Hq, D = q.shape
        Hkv = k.shape[1]
        out = np.zeros((B, q_len, Hq))
        for b in range(B):
            for i in range(q_len):
                Lb = int(kv_lens[b])
                n = Lb if mistake == "energy_rows_no_causal" else oracle.visible(Lb, q_len, i, causal)
                for h in range(Hq):
                    kvh = h % Hkv if mistake == "energy_rows_gqa_modulo" else h // (Hq // Hkv)
                    out[b, i, h] = energy(q[b, i, h], k[b, kvh, :n], v[b, kvh, :n], scale, zeta[b, i, h])
        return out
    return energy_rows


ATTEND_MISTAKES = ["no_scale", "sign", "kv_swapped", "gqa_modulo", "causal_off_by_one",
                   "causal_ignored", "lse_log2", "lse_drops_max", "unnormalised", "no_max_shift"]
MERGE_MISTAKES = ["merge_no_rescale_o", "merge_inverted_weight"]
ENERGY_MISTAKES = ["energy_no_zeta", "energy_scaled_zeta"]
PAGING_MISTAKES = ["page_strides_swapped", "page_quotient_remainder_swapped", "page_ignores_table"]
ENERGY_ROWS_MISTAKES = ["energy_rows_no_causal", "energy_rows_gqa_modulo"]
ANCHOR_MISTAKES = ["anchor_after_block", "anchor_block_not_causal"]


def _anchor_factory(attend, mistake):
    def attend_anchor_blocks(q, ka, va, kb, vb, scale, blocks=None):
        N, Lb, Hq, D = q.shape
        A = ka.shape[1]
        O = np.zeros(q.shape); lse = np.zeros((N, Lb, Hq))
        for b in range(N):
            if mistake == "anchor_after_block":
                kc = np.concatenate([kb[b], ka], axis=1)[None]; vc = np.concatenate([vb[b], va], axis=1)[None]
            else:
                kc = np.concatenate([ka, kb[b]], axis=1)[None]; vc = np.concatenate([va, vb[b]], axis=1)[None]
            causal = mistake != "anchor_block_not_causal"
            o, l = attend(q[b][None], kc, vc, [A + Lb], scale, causal)
            O[b], lse[b] = o[0], l[0]
        return O, lse
    return attend_anchor_blocks


def _impl(mistake):
    att = _attend_factory(mistake if mistake in ATTEND_MISTAKES else None)
    gather = _gather_factory(mistake)
    energy = _energy_factory(mistake)
    return types.SimpleNamespace(
        attend=att,
        attend_bifurcated=_bif_factory(att),
        attend_anchor_blocks=_anchor_factory(att, mistake),
        gather=gather,
        attend_paged=_attend_paged_factory(att, gather),
        energy=energy,
        energy_rows=_energy_rows_factory(energy, mistake),
        chunk_partial=oracle.chunk_partial,
        merge=_merge_factory(mistake),
        finalize=oracle.finalize,
    )


def test_faithful_variant_passes_all_pins():
    """The loop-based variant with no mistake passes every pin (so the mutants
    below fail because of their mistake, not because of the harness)."""
    impl = _impl(None)
    for pin in pins.ALL_PINS:
        pin(impl)


@pytest.mark.parametrize("mistake", ATTEND_MISTAKES + MERGE_MISTAKES + ENERGY_MISTAKES +
                         PAGING_MISTAKES + ENERGY_ROWS_MISTAKES + ANCHOR_MISTAKES)
def test_pins_catch_planted_mistake(mistake):
    impl = _impl(mistake)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, ValueError, FloatingPointError, OverflowError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {mistake!r}"
