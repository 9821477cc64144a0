"""Pins for the fp64 oracle: checks against facts that do not come from the oracle.

Each ``pin_*`` takes an implementation namespace ``impl`` (the real ``oracle``
module, or a deliberately broken variant built in test_oracle_mutants.py) and
raises AssertionError when ``impl`` disagrees with:

* hand-worked closed-form examples (tests/golden/hand_worked.json);
* brute-force softmax written with pure-Python loops and math.fsum;
* library routines: torch's fp64 CPU scaled_dot_product_attention and
  torch/scipy logsumexp;
* closed forms (single key, identical keys, zero query, two keys, huge
  logits) and invariants (row permutation, affine V, GQA as repeated MHA,
  causal block as truncated decode);
* the energy view: central finite differences of F(zeta) give O;
* associativity: random chunkings and random merge trees reproduce O and lse;
* bifurcation: prefix/suffix merge equals attention over the concatenation;
* paging: hand-worked paged caches, and pools written by a pure-Python
  scatter (both page layouts, shared pages) resolve to the dense cache;
* row energies: F(0) is the row's logsumexp, and closed forms for constant
  values and a single key;
* anchor-block context encoding: brute force on tiny inputs, and for two
  blocks the second block's result equals global causal attention.
"""
from __future__ import annotations

import json
import math
import os
import random
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.json")


def _num(x) -> float:
    if isinstance(x, (int, float)):
        return float(x)
    x = x.strip()
    if x.startswith("ln "):
        return math.log(float(Fraction(x[3:])))
    return float(Fraction(x))


def _ln_of(x: str) -> float:
    f = Fraction(x)
    return -math.inf if f == 0 else math.log(float(f))


def _close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    inf_a, inf_b = np.isinf(a), np.isinf(b)
    assert (inf_a == inf_b).all() and (a[inf_a] == b[inf_b]).all(), f"{what}: infinities differ {a} vs {b}"
    fin = ~inf_a
    assert not np.isnan(a[fin]).any(), f"{what}: NaN in {a}"
    assert np.allclose(a[fin], b[fin], rtol=rtol, atol=atol), f"{what}: {a} vs {b}"


# ----------------------------------------------------------------------------
# Golden, hand-worked examples
# ----------------------------------------------------------------------------
def pin_golden(impl):
    with open(GOLDEN) as f:
        g = json.load(f)
    for ex in g["decode"]:
        q = np.array([[[_num(x) for x in row] for row in tok] for tok in ex["q"]])[None]
        k = np.array([[[_num(x) for x in row] for row in hd] for hd in ex["k"]])[None]
        v = np.array([[[_num(x) for x in row] for row in hd] for hd in ex["v"]])[None]
        O, lse = impl.attend(q, k, v, [ex["kv_len"]], ex["scale"], ex["causal"])
        want_O = np.array([[[_num(x) for x in row] for row in tok] for tok in ex["O"]])[None]
        want_lse = np.array([[_ln_of(x) for x in tok] for tok in ex["lse_ln_of"]])[None]
        _close(O, want_O, what=ex["name"] + " O")
        _close(lse, want_lse, what=ex["name"] + " lse")
    for ex in g["merge"]:
        s = np.array([_num(x) for x in ex["s"]])
        v = np.array([[_num(x) for x in row] for row in ex["v"]])
        c = ex["split"]
        pa = impl.chunk_partial(s[:c], v[:c])
        pb = impl.chunk_partial(s[c:], v[c:])
        for p, w, nm in ((pa, ex["a"], "a"), (pb, ex["b"], "b")):
            _close(p[0], _ln_of(w["m_ln_of"]), what=f"{ex['name']} m_{nm}")
            _close(p[1], _num(w["l"]), what=f"{ex['name']} l_{nm}")
            _close(p[2], [_num(x) for x in w["o"]], what=f"{ex['name']} o_{nm}")
        pm = impl.merge(pa, pb)
        w = ex["merged"]
        _close(pm[0], _ln_of(w["m_ln_of"]), what="merged m")
        _close(pm[1], _num(w["l"]), what="merged l")
        _close(pm[2], [_num(x) for x in w["o"]], what="merged o")
        O, lse = impl.finalize(pm)
        _close(O, [_num(x) for x in ex["O"]], what="finalized O")
        _close(lse, _ln_of(ex["lse_ln_of"]), what="finalized lse")


# ----------------------------------------------------------------------------
# Brute force with pure-Python loops (tiny inputs only)
# ----------------------------------------------------------------------------
def _random_case(rng: np.random.Generator, causal: bool):
    B = int(rng.integers(1, 3))
    q_len = int(rng.integers(1, 4)) if causal else 1
    Hkv = int(rng.integers(1, 3))
    G = int(rng.integers(1, 4))
    Hq = Hkv * G
    D = int(rng.integers(1, 9))
    L = int(rng.integers(q_len, 40))
    lens = rng.integers(q_len if causal else 0, L + 1, size=B)
    q = rng.standard_normal((B, q_len, Hq, D)) * 1.5
    k = rng.standard_normal((B, Hkv, L, D))
    v = rng.standard_normal((B, Hkv, L, D))
    scale = float(rng.uniform(0.2, 1.5))
    return q, k, v, lens, scale


def _brute(q, k, v, lens, scale, causal):
    B, q_len, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    O = np.zeros(q.shape)
    lse = np.zeros((B, q_len, Hq))
    for b in range(B):
        for i in range(q_len):
            n = int(lens[b]) - q_len + i + 1 if causal else int(lens[b])
            for h in range(Hq):
                kv = h // G
                s = [scale * math.fsum(float(q[b, i, h, j]) * float(k[b, kv, t, j]) for j in range(D))
                     for t in range(n)]
                if n == 0:
                    lse[b, i, h] = -math.inf
                    continue
                M = max(s)
                Z = math.fsum(math.exp(x - M) for x in s)
                lse[b, i, h] = M + math.log(Z)
                for j in range(D):
                    O[b, i, h, j] = math.fsum(math.exp(s[t] - M) / Z * float(v[b, kv, t, j])
                                              for t in range(n))
    return O, lse


def pin_brute_force(impl, n_cases: int = 12, seed: int = 7):
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        causal = bool(c % 2)
        q, k, v, lens, scale = _random_case(rng, causal)
        O, lse = impl.attend(q, k, v, lens, scale, causal)
        Ob, lb = _brute(q, k, v, lens, scale, causal)
        _close(O, Ob, rtol=1e-11, atol=1e-12, what=f"brute case {c} O")
        _close(lse, lb, rtol=1e-12, atol=1e-12, what=f"brute case {c} lse")


# ----------------------------------------------------------------------------
# Library routines
# ----------------------------------------------------------------------------
def pin_library(impl, n_cases: int = 8, seed: int = 11):
    import torch
    import scipy.special
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        causal = bool(c % 2)
        q, k, v, lens, scale = _random_case(rng, causal)
        B, q_len, Hq, D = q.shape
        Hkv, L = k.shape[1], k.shape[2]
        G = Hq // Hkv
        O, lse = impl.attend(q, k, v, lens, scale, causal)
        tq = torch.from_numpy(q).permute(0, 2, 1, 3).contiguous()          # [B,Hq,q_len,D]
        tk = torch.from_numpy(k).repeat_interleave(G, dim=1).contiguous()  # [B,Hq,L,D]
        tv = torch.from_numpy(v).repeat_interleave(G, dim=1).contiguous()
        t = torch.arange(L)
        for b in range(B):
            lim = torch.tensor([(int(lens[b]) - q_len + i + 1) if causal else int(lens[b])
                                for i in range(q_len)])
            mask = t[None, :] < lim[:, None]                                 # [q_len, L]
            if not mask.any(dim=1).all():
                continue  # sdpa yields NaN for rows with no key; closed forms cover them
            ref = torch.nn.functional.scaled_dot_product_attention(
                tq[b:b + 1], tk[b:b + 1], tv[b:b + 1], attn_mask=mask[None, None], scale=scale)
            _close(O[b], ref[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12,
                   what=f"sdpa case {c}")
            logits = scale * (tq[b] @ tk[b].transpose(-1, -2))
            logits = logits.masked_fill(~mask[None], -math.inf)
            ref_lse = torch.logsumexp(logits, dim=-1).permute(1, 0).numpy()
            _close(lse[b], ref_lse, rtol=1e-12, atol=1e-12, what=f"torch lse case {c}")
            sp = scipy.special.logsumexp(logits.numpy(), axis=-1).T
            _close(lse[b], sp, rtol=1e-12, atol=1e-12, what=f"scipy lse case {c}")


# ----------------------------------------------------------------------------
# Closed forms
# ----------------------------------------------------------------------------
def pin_closed_forms(impl, seed: int = 3):
    rng = np.random.default_rng(seed)
    D = 6
    # single key: O = v0, lse = s0
    q = rng.standard_normal((1, 1, 1, D)); k = rng.standard_normal((1, 1, 1, D))
    v = rng.standard_normal((1, 1, 1, D)); sc = 0.7
    O, lse = impl.attend(q, k, v, [1], sc)
    _close(O[0, 0, 0], v[0, 0, 0], what="single key O")
    _close(lse[0, 0, 0], sc * float(q[0, 0, 0] @ k[0, 0, 0]), what="single key lse")
    # identical keys: O = mean V, lse = s + ln L
    L = 9
    k = np.repeat(rng.standard_normal((1, 1, 1, D)), L, axis=2)
    v = rng.standard_normal((1, 1, L, D))
    O, lse = impl.attend(q, k, v, [L], sc)
    _close(O[0, 0, 0], v[0, 0].mean(axis=0), what="identical keys O")
    _close(lse[0, 0, 0], sc * float(q[0, 0, 0] @ k[0, 0, 0]) + math.log(L), what="identical keys lse")
    # zero query: O = mean V, lse = ln L
    k = rng.standard_normal((1, 1, L, D))
    O, lse = impl.attend(np.zeros((1, 1, 1, D)), k, v, [L], sc)
    _close(O[0, 0, 0], v[0, 0].mean(axis=0), what="zero query O")
    _close(lse[0, 0, 0], math.log(L), what="zero query lse")
    # two keys: lse = logaddexp(s0, s1), O = sigma(s0 - s1) v0 + sigma(s1 - s0) v1
    k = rng.standard_normal((1, 1, 2, D)); v = rng.standard_normal((1, 1, 2, D))
    s0 = sc * float(q[0, 0, 0] @ k[0, 0, 0]); s1 = sc * float(q[0, 0, 0] @ k[0, 0, 1])
    O, lse = impl.attend(q, k, v, [2], sc)
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    _close(lse[0, 0, 0], np.logaddexp(s0, s1), what="two keys lse")
    _close(O[0, 0, 0], sig(s0 - s1) * v[0, 0, 0] + sig(s1 - s0) * v[0, 0, 1], what="two keys O")
    # huge logits: s = (1000, 1000 - ln 3) -> lse = 1000 + ln(4/3), weights (3/4, 1/4)
    q = np.zeros((1, 1, 1, 2)); q[..., 0] = 1.0
    k = np.array([[[[1000.0, 0.0], [1000.0 - math.log(3.0), 0.0]]]])
    v = np.array([[[[4.0, 0.0], [0.0, 4.0]]]])
    O, lse = impl.attend(q, k, v, [2], 1.0)
    _close(lse[0, 0, 0], 1000.0 + math.log(4.0 / 3.0), what="huge logits lse")
    _close(O[0, 0, 0], [3.0, 1.0], what="huge logits O")


# ----------------------------------------------------------------------------
# Invariants
# ----------------------------------------------------------------------------
def pin_invariants(impl, seed: int = 5):
    rng = np.random.default_rng(seed)
    B, Hkv, G, D, L = 2, 2, 3, 5, 23
    q = rng.standard_normal((B, 1, Hkv * G, D)); k = rng.standard_normal((B, Hkv, L, D))
    v = rng.standard_normal((B, Hkv, L, D)); lens = [L, 17]; sc = 0.6
    O, lse = impl.attend(q, k, v, lens, sc)
    # permuting the visible K/V rows together changes nothing
    for b in range(B):
        n = lens[b]
        perm = rng.permutation(n)
        kp, vp = k.copy(), v.copy()
        kp[b, :, :n] = k[b][:, perm]; vp[b, :, :n] = v[b][:, perm]
        O2, lse2 = impl.attend(q, kp, vp, lens, sc)
        _close(O2, O, rtol=1e-12, atol=1e-13, what="permutation O")
        _close(lse2, lse, rtol=1e-12, atol=1e-13, what="permutation lse")
    # V -> a V + c  gives  O -> a O + c, lse unchanged
    a, c = -1.7, rng.standard_normal(D)
    O3, lse3 = impl.attend(q, k, a * v + c, lens, sc)
    _close(O3, a * O + c, rtol=1e-12, atol=1e-12, what="affine V O")
    _close(lse3, lse, what="affine V lse")
    # GQA equals MHA with each KV head repeated for its group (head h reads h // G)
    k_rep = np.repeat(k, G, axis=1); v_rep = np.repeat(v, G, axis=1)
    O4, lse4 = impl.attend(q, k_rep, v_rep, lens, sc)
    _close(O4, O, what="GQA = repeated MHA O")
    _close(lse4, lse, what="GQA = repeated MHA lse")
    # padding past L_b is never read
    kn, vn = k.copy(), v.copy()
    kn[1, :, lens[1]:] = np.nan; vn[1, :, lens[1]:] = np.nan
    O5, lse5 = impl.attend(q, kn, vn, lens, sc)
    _close(O5, O, what="NaN padding O")
    _close(lse5, lse, what="NaN padding lse")


def pin_causal_truncation(impl, seed: int = 9):
    rng = np.random.default_rng(seed)
    B, q_len, Hkv, G, D, L = 2, 4, 2, 2, 5, 30
    q = rng.standard_normal((B, q_len, Hkv * G, D)); k = rng.standard_normal((B, Hkv, L, D))
    v = rng.standard_normal((B, Hkv, L, D)); lens = [L, 11]; sc = 0.45
    O, lse = impl.attend(q, k, v, lens, sc, True)
    for b in range(B):
        for i in range(q_len):
            n = lens[b] - q_len + i + 1
            Oi, li = impl.attend(q[b:b + 1, i:i + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], [n], sc)
            _close(O[b, i], Oi[0, 0], what=f"causal b{b} i{i} O")
            _close(lse[b, i], li[0, 0], what=f"causal b{b} i{i} lse")


# ----------------------------------------------------------------------------
# Energy view: O is the zeta-gradient of F at zeta = 0
# ----------------------------------------------------------------------------
def pin_energy_gradient(impl, seed: int = 13, h: float = 1e-5):
    rng = np.random.default_rng(seed)
    for L, D, sc in ((1, 3, 1.0), (7, 4, 0.5), (33, 8, 0.35)):
        q = rng.standard_normal(D); k = rng.standard_normal((L, D)); v = rng.standard_normal((L, D))
        O, lse = impl.attend(q[None, None, None], k[None, None], v[None, None], [L], sc)
        F0 = impl.energy(q, k, v, sc, np.zeros(D))
        _close(F0, lse[0, 0, 0], what="F(0) = lse")
        grad = np.empty(D)
        for j in range(D):
            e = np.zeros(D); e[j] = h
            grad[j] = (impl.energy(q, k, v, sc, e) - impl.energy(q, k, v, sc, -e)) / (2 * h)
        _close(grad, O[0, 0, 0], rtol=1e-7, atol=1e-7, what="dF/dzeta = O")


# ----------------------------------------------------------------------------
# Associativity: any chunking, any merge tree
# ----------------------------------------------------------------------------
def _random_tree_merge(impl, parts, rnd: random.Random):
    parts = list(parts)
    while len(parts) > 1:
        i = rnd.randrange(len(parts) - 1)
        parts[i:i + 2] = [impl.merge(parts[i], parts[i + 1])]
    return parts[0]


def pin_chunk_merge(impl, n_cases: int = 25, seed: int = 17):
    rng = np.random.default_rng(seed)
    rnd = random.Random(seed)
    for c in range(n_cases):
        L = int(rng.integers(1, 200)); D = int(rng.integers(1, 9)); sc = float(rng.uniform(0.1, 2))
        q = rng.standard_normal(D) * 2; k = rng.standard_normal((L, D)); v = rng.standard_normal((L, D))
        if c % 5 == 0:
            k[rng.integers(0, L)] = 40.0 * q / np.linalg.norm(q) / sc  # dominant key
        O, lse = impl.attend(q[None, None, None], k[None, None], v[None, None], [L], sc)
        s = sc * (k @ q)
        n_cut = int(rng.integers(0, min(L, 12)))
        cuts = sorted(rng.choice(np.arange(0, L + 1), size=n_cut, replace=True).tolist())
        bounds = [0] + cuts + [L]  # repeated cuts give empty chunks (identity records)
        parts = [impl.chunk_partial(s[a:b], v[a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
        Om, lm = impl.finalize(_random_tree_merge(impl, parts, rnd))
        _close(Om, O[0, 0, 0], rtol=1e-11, atol=1e-12, what=f"chunk merge case {c} O")
        _close(lm, lse[0, 0, 0], rtol=1e-12, atol=1e-12, what=f"chunk merge case {c} lse")
    # the identity record is neutral on both sides, and two identities stay identity
    ident = impl.chunk_partial(np.zeros(0), np.zeros((0, 3)))
    p = impl.chunk_partial(np.array([0.3, -1.0]), np.ones((2, 3)))
    for x in (impl.merge(ident, p), impl.merge(p, ident)):
        _close(x[0], p[0], what="identity m"); _close(x[1], p[1], what="identity l")
        _close(x[2], p[2], what="identity o")
    e = impl.finalize(impl.merge(ident, ident))
    _close(e[0], np.zeros(3), what="empty O"); _close(e[1], -math.inf, what="empty lse")


# ----------------------------------------------------------------------------
# Bifurcation: prefix + per-sample suffix
# ----------------------------------------------------------------------------
def pin_bifurcated(impl, seed: int = 19):
    rng = np.random.default_rng(seed)
    S, Hkv, G, D, Lp, Ls = 3, 2, 2, 6, 21, 5
    q = rng.standard_normal((S, Hkv * G, D)); kp = rng.standard_normal((Hkv, Lp, D))
    vp = rng.standard_normal((Hkv, Lp, D)); ks = rng.standard_normal((S, Hkv, Ls, D))
    vs = rng.standard_normal((S, Hkv, Ls, D)); sc = 0.4
    O, lse = impl.attend_bifurcated(q, kp, vp, ks, vs, sc)
    for s in range(S):
        kc = np.concatenate([kp, ks[s]], axis=1)[None]; vc = np.concatenate([vp, vs[s]], axis=1)[None]
        Oc, lc = impl.attend(q[s][None, None], kc, vc, [Lp + Ls], sc)
        _close(O[s], Oc[0, 0], what="bifurcated = concatenation O")
        _close(lse[s], lc[0, 0], what="bifurcated = concatenation lse")
        for h in range(Hkv * G):
            kvh = h // G
            sp = sc * (kp[kvh] @ q[s, h]); ss = sc * (ks[s, kvh] @ q[s, h])
            Om, lm = impl.finalize(impl.merge(impl.chunk_partial(sp, vp[kvh]),
                                              impl.chunk_partial(ss, vs[s, kvh])))
            _close(Om, O[s, h], what="bifurcated = prefix (+) suffix O")
            _close(lm, lse[s, h], what="bifurcated = prefix (+) suffix lse")


# ----------------------------------------------------------------------------
# Paged caches
# ----------------------------------------------------------------------------
def _elem(x) -> float:
    return math.nan if x == "nan" else _num(x)


def pin_paged_golden(impl):
    with open(GOLDEN) as f:
        g = json.load(f)
    for ex in g["paged"]:
        kp = np.array([_elem(x) for x in ex["k_pool"]])
        vp = np.array([_elem(x) for x in ex["v_pool"]])
        table = np.array(ex["table"], dtype=np.int32)
        L, Lm, Hkv, D = ex["kv_len"], ex["L_max"], ex["Hkv"], ex["D"]
        geo = (ex["page_size"], ex["page_stride"], ex["head_stride"], ex["token_stride"])
        dense = impl.gather(kp, table, [L], *geo, Hkv, D, Lm)
        want = np.array([[[_num(x) for x in row] for row in hd] for hd in ex["dense_k"]])
        _close(dense[0, :, :L], want, what=ex["name"] + " gathered K")
        assert np.isnan(dense[0, :, L:]).all(), ex["name"] + ": positions past L must stay unread"
        q = np.array(ex["q"])[None]
        O, lse = impl.attend_paged(q, kp, vp, table, [L], ex["scale"], page_size=geo[0],
                                   page_stride=geo[1], head_stride=geo[2], token_stride=geo[3],
                                   num_kv_heads=Hkv, L_max=Lm)
        want_O = np.array([[[_num(x) for x in row] for row in tok] for tok in ex["O"]])[None]
        want_lse = np.array([[_ln_of(x) for x in tok] for tok in ex["lse_ln_of"]])[None]
        _close(O, want_O, what=ex["name"] + " O")
        _close(lse, want_lse, what=ex["name"] + " lse")


def _scatter_by_loops(k, lens, P, layout, order, share_first_page):
    """Pool and block table written element by element (independent of the
    oracle's vectorised gather).  Physical page numbers follow ``order``."""
    B, Hkv, _, D = k.shape
    if layout == "head_major":
        ps, hs, ts = Hkv * P * D, P * D, D
    else:
        ps, hs, ts = P * Hkv * D, D, Hkv * D
    pages_per_seq = max(1, -(-k.shape[2] // P))
    table = [[-1] * pages_per_seq for _ in range(B)]
    nxt = 0
    for b in range(B):
        for j in range(-(-int(lens[b]) // P)):
            if share_first_page and b > 0 and j == 0:
                table[b][j] = table[0][0]
                continue
            table[b][j] = int(order[nxt])
            nxt += 1
    pool = [math.nan] * (len(order) * ps)
    for b in range(B):
        for t in range(int(lens[b])):
            p = table[b][t // P]
            for h in range(Hkv):
                for e in range(D):
                    pool[p * ps + h * hs + (t % P) * ts + e] = float(k[b, h, t, e])
    return np.array(pool), np.array(table, dtype=np.int32), (P, ps, hs, ts)


def pin_paged_scatter(impl, n_cases: int = 8, seed: int = 23):
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        layout = ("head_major", "token_major")[c % 2]
        causal = c % 4 >= 2
        share = c % 3 == 0
        B = int(rng.integers(1, 4)); Hkv = int(rng.integers(1, 3)); G = int(rng.integers(1, 3))
        D = int(rng.integers(1, 5)); P = 1 << int(rng.integers(0, 4))
        q_len = 2 if causal else 1
        Lm = int(rng.integers(q_len, 30))
        lens = rng.integers(q_len if causal else 0, Lm + 1, size=B)
        if share:
            lens = np.maximum(lens, min(P, Lm))
        k = rng.standard_normal((B, Hkv, Lm, D)); v = rng.standard_normal((B, Hkv, Lm, D))
        if share:  # every sequence starts with sequence 0's first page
            n0 = min(P, int(lens.min()))
            k[1:, :, :n0] = k[0, :, :n0]; v[1:, :, :n0] = v[0, :, :n0]
            share = n0 == P
        q = rng.standard_normal((B, q_len, Hkv * G, D))
        n_pages = sum(-(-int(L) // P) for L in lens) + 3
        order = rng.permutation(n_pages)
        kp, table, geo = _scatter_by_loops(k, lens, P, layout, order, share)
        vp, _, _ = _scatter_by_loops(v, lens, P, layout, order, share)
        dense = impl.gather(kp, table, lens, *geo, Hkv, D, Lm)
        for b in range(B):
            _close(dense[b, :, :lens[b]], k[b, :, :lens[b]], what=f"paged case {c} gather b={b}")
            assert np.isnan(dense[b, :, lens[b]:]).all(), f"paged case {c}: read past L_b"
        O, lse = impl.attend_paged(q, kp, vp, table, lens, 0.7, page_size=geo[0],
                                   page_stride=geo[1], head_stride=geo[2], token_stride=geo[3],
                                   num_kv_heads=Hkv, L_max=Lm, causal=causal)
        Od, ld = impl.attend(q, k, v, lens, 0.7, causal)
        _close(O, Od, what=f"paged case {c} O"); _close(lse, ld, what=f"paged case {c} lse")


# ----------------------------------------------------------------------------
# Row energies F(zeta) of a decode call
# ----------------------------------------------------------------------------
def pin_energy_rows(impl, seed: int = 29):
    rng = np.random.default_rng(seed)
    B, q_len, Hkv, G, D, Lm = 3, 2, 2, 3, 5, 17
    q = rng.standard_normal((B, q_len, Hkv * G, D)); k = rng.standard_normal((B, Hkv, Lm, D))
    v = rng.standard_normal((B, Hkv, Lm, D)); lens = np.array([17, 2, 9]); sc = 0.6
    _, lse = impl.attend(q, k, v, lens, sc, True)
    F0 = impl.energy_rows(q, k, v, lens, sc, np.zeros(q.shape), True)
    _close(F0, lse, what="F(0) = lse for every row")
    # Constant values u per KV head: F(zeta) = lse + zeta . u
    u = rng.standard_normal((B, Hkv, D))
    vc = np.repeat(u[:, :, None, :], Lm, axis=2)
    zeta = rng.standard_normal(q.shape)
    Fz = impl.energy_rows(q, k, vc, lens, sc, zeta, True)
    want = lse + np.einsum("bihd,bhd->bih", zeta, np.repeat(u, G, axis=1))
    _close(Fz, want, rtol=1e-12, atol=1e-12, what="F(zeta) with constant V")
    # One visible key per row: F(zeta) = scale q.k_0 + zeta.v_0
    l1 = np.array([1, 1, 1])
    F1 = impl.energy_rows(q[:, :1], k, v, l1, sc, zeta[:, :1], False)
    for b in range(B):
        for h in range(Hkv * G):
            s0 = sc * float(q[b, 0, h] @ k[b, h // G, 0]) + float(zeta[b, 0, h] @ v[b, h // G, 0])
            _close(F1[b, 0, h], s0, what="single-key F(zeta)")


# ----------------------------------------------------------------------------
# Anchor-block context encoding (Star Attention, phase 1)
# ----------------------------------------------------------------------------
def _brute_anchor(q, ka, va, kb, vb, scale):
    N, Lb, Hq, D = q.shape
    Hkv, A, _ = ka.shape
    G = Hq // Hkv
    O = np.zeros(q.shape); lse = np.zeros((N, Lb, Hq))
    for b in range(N):
        for i in range(Lb):
            for h in range(Hq):
                kv = h // G
                keys = [ka[kv, t] for t in range(A)] + [kb[b, kv, t] for t in range(i + 1)]
                vals = [va[kv, t] for t in range(A)] + [vb[b, kv, t] for t in range(i + 1)]
                s = [scale * math.fsum(float(q[b, i, h, j]) * float(k[j]) for j in range(D)) for k in keys]
                M = max(s); Z = math.fsum(math.exp(x - M) for x in s)
                lse[b, i, h] = M + math.log(Z)
                for j in range(D):
                    O[b, i, h, j] = math.fsum(math.exp(s[t] - M) / Z * float(vals[t][j]) for t in range(len(s)))
    return O, lse


def pin_anchor_blocks(impl, seed: int = 31):
    rng = np.random.default_rng(seed)
    # brute force on tiny inputs
    for (N, Lb, Hkv, G, D, A) in ((2, 3, 1, 2, 3, 4), (3, 2, 2, 1, 2, 1), (1, 4, 1, 1, 5, 0)):
        q = rng.standard_normal((N, Lb, Hkv * G, D)); ka = rng.standard_normal((Hkv, A, D))
        va = rng.standard_normal((Hkv, A, D)); kb = rng.standard_normal((N, Hkv, Lb, D))
        vb = rng.standard_normal((N, Hkv, Lb, D))
        O, lse = impl.attend_anchor_blocks(q, ka, va, kb, vb, 0.6)
        Ob, lb = _brute_anchor(q, ka, va, kb, vb, 0.6)
        _close(O, Ob, what="anchor blocks vs brute force O")
        _close(lse, lb, what="anchor blocks vs brute force lse")
    # With two blocks, block 1 with block 0 as its anchor sees exactly what
    # global causal attention over the whole context shows it.
    Lb, Hkv, G, D = 6, 2, 2, 4
    q = rng.standard_normal((1, 2 * Lb, Hkv * G, D)); k = rng.standard_normal((1, Hkv, 2 * Lb, D))
    v = rng.standard_normal((1, Hkv, 2 * Lb, D))
    Og, lg = impl.attend(q, k, v, [2 * Lb], 0.5, True)
    O1, l1 = impl.attend_anchor_blocks(q[0, Lb:][None], k[0, :, :Lb], v[0, :, :Lb],
                                       k[0, :, Lb:][None], v[0, :, Lb:][None], 0.5)
    _close(O1[0], Og[0, Lb:], what="block 1 with anchor = global causal O")
    _close(l1[0], lg[0, Lb:], what="block 1 with anchor = global causal lse")


ALL_PINS = [pin_golden, pin_brute_force, pin_library, pin_closed_forms, pin_invariants,
            pin_causal_truncation, pin_energy_gradient, pin_chunk_merge, pin_bifurcated,
            pin_paged_golden, pin_paged_scatter, pin_energy_rows, pin_anchor_blocks]
