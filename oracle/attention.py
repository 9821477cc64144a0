"""CPU fp64 oracle for exact softmax attention decoding over a KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
does.  It shares no code with the HIP library: it widens bfloat16 bits itself
and computes everything in float64 with plain numpy (matrix products are the
only library primitive used as a step).

What it computes, and where that is stated:

* ``attend`` -- the plain definition of attention, S = Q K^T / sqrt(d_k),
  P = softmax(S), O = P V ("attention acceleration" concept page, section
  "technical principles" 1, self-attention recap), for one query row at a time,
  with the softmax taken in two passes (max, then the sum of exponentials of
  the shifted logits, whose log gives the logsumexp).  The per-row statistics
  m = max x and l = sum e^(x - m) are the ones the same page defines in its
  section 2.1 (tiling and online softmax).
* ``energy`` -- Tree Attention's scalar energy F(K, Q, V, zeta), whose
  gradient in the auxiliary variable zeta at zeta = 0 is the attention output
  (Tree Attention article, section "an energy view of attention").  The page
  lost the decode formula in extraction; the reading used here is
  F(zeta) = ln sum_t exp(scale * q.k_t + zeta.v_t), the logsumexp form the
  article's associativity remark relies on.  F(0) is the row's logsumexp.
* ``energy_rows`` -- F(zeta) for every row of a decode call, one zeta
  vector per row, each row over its own visible keys.
* ``chunk_partial`` / ``merge`` / ``finalize`` -- the per-chunk statistics
  (m, l, o) with o the unnormalised partial output, and the combination rule
  m = max(m_a, m_b), l = l_a e^(m_a - m) + l_b e^(m_b - m), same for o
  (concept page section 2.1, the m_new / l_new / O_new updates written in
  unnormalised form).  Because max and logsumexp are associative (Tree
  Attention article, same section), any chunking and any merge order gives
  the same result; Star Attention's phase 2 (query encoding and token
  generation) aggregates exactly these statistics across hosts.
* ``attend_bifurcated`` -- Bifurcated Attention (TL;DR) splits decode
  attention into one GEMM over the shared prefilled KV and one over each
  sample's decoded KV, as an exact rewrite.  The oracle therefore does not
  split: it attends each sample over the concatenation [prefix ; suffix].
* ``attend_anchor_blocks`` -- Star Attention's context encoding (phase 1 on
  the Star Attention page): the context is cut into blocks and every block
  but the first is processed with the first block, the anchor, placed in
  front of it.  Reading fixed here where the page is silent: within the
  block attention is causal, and every anchor key is visible to every query
  of the block (the anchor precedes it), so block b's query token i attends
  over [anchor ; block b] causally, i.e. ``attend`` with q_len = Lb over the
  concatenation.

Conventions fixed where the pages are silent:
  * natural-log logsumexp of the *scaled* logits;
  * GQA: query head h reads KV head h // (Hq // Hkv);
  * causal query blocks: kv_lens[b] counts the q_len new tokens, and query
    token i (0-based) sees keys t <= kv_lens[b] - q_len + i;
  * a row that sees no key has O = 0 and lse = -inf (the identity of the
    merge is (m, l, o) = (-inf, 0, 0)).
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

SLAB = 65536


def _widen(a: np.ndarray) -> np.ndarray:
    """float64 copy of an array given as floats or as uint16 bfloat16 bits."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def visible(L_b: int, q_len: int, i: int, causal: bool) -> int:
    """Number of keys (a prefix of the cache) that query token i sees."""
    n = L_b - q_len + i + 1 if causal else L_b
    return max(0, min(int(L_b), int(n)))


# ----------------------------------------------------------------------------
# Plain attention (the definition)
# ----------------------------------------------------------------------------
def attend_row(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> Tuple[np.ndarray, float]:
    """O and lse of one query row q[D] against keys k[n, D] and values v[n, D]."""
    q, k, v = _widen(q), _widen(k), _widen(v)
    n = k.shape[0]
    if n == 0:
        return np.zeros(v.shape[1]), -math.inf
    s = scale * (k @ q)
    M = s.max()
    lse = M + math.log(np.exp(s - M).sum())
    p = np.exp(s - lse)
    return p @ v, lse


def attend(q: np.ndarray, k: np.ndarray, v: Optional[np.ndarray], kv_lens, scale: float,
           causal: bool = False, rows: Optional[Iterable[Tuple[int, int, int]]] = None,
           slab: int = SLAB):
    """Plain attention for a decode call.

    q [B][q_len][Hq][D]; k, v [B][Hkv][L_max][D] (floats or bf16 bits);
    kv_lens[b] = cached length of sequence b.  With ``v`` None only the
    logsumexp is produced.  ``rows`` restricts the work to the listed
    (b, i, h) rows (sampled checks on caches too large to do whole).

    Returns (O [B][q_len][Hq][D] or None, lse [B][q_len][Hq]) in float64;
    rows that were not requested hold NaN.
    """
    B, q_len, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    lens = np.asarray(kv_lens, dtype=np.int64).reshape(B)
    O = np.full((B, q_len, Hq, D), np.nan) if v is not None else None
    lse = np.full((B, q_len, Hq), np.nan)
    if rows is None:
        want = {(b, kvh): [(i, h) for i in range(q_len) for h in range(kvh * G, (kvh + 1) * G)]
                for b in range(B) for kvh in range(Hkv)}
    else:
        want = {}
        for (b, i, h) in rows:
            want.setdefault((b, h // G), []).append((i, h))
    for (b, kvh), rws in want.items():
        Lb = int(lens[b])
        Qr = np.stack([_widen(q[b, i, h]) for (i, h) in rws])  # [R, D]
        nvis = np.array([visible(Lb, q_len, i, causal) for (i, _) in rws])
        n_all = int(nvis.max()) if len(nvis) else 0
        # pass 1: every visible logit of every row
        S = np.full((len(rws), n_all), -np.inf)
        for t0 in range(0, n_all, slab):
            t1 = min(n_all, t0 + slab)
            S[:, t0:t1] = scale * (Qr @ _widen(k[b, kvh, t0:t1]).T)
        for r, n in enumerate(nvis):
            S[r, n:] = -np.inf
        # pass 2: max, logsumexp, weights
        M = np.where(nvis > 0, S.max(axis=1, initial=-np.inf), 0.0)
        lrow = np.exp(S - M[:, None]).sum(axis=1)
        with np.errstate(divide="ignore"):
            lr = np.where(nvis > 0, M + np.log(lrow), -np.inf)
        for r, (i, h) in enumerate(rws):
            lse[b, i, h] = lr[r]
        if v is not None:
            acc = np.zeros((len(rws), v.shape[-1]))
            Pw = np.exp(S - np.where(nvis > 0, lr, 0.0)[:, None])
            Pw[nvis == 0] = 0.0
            for t0 in range(0, n_all, slab):
                t1 = min(n_all, t0 + slab)
                acc += Pw[:, t0:t1] @ _widen(v[b, kvh, t0:t1])
            for r, (i, h) in enumerate(rws):
                O[b, i, h] = acc[r]
    return O, lse


def attend_bifurcated(q: np.ndarray, kp: np.ndarray, vp: np.ndarray, ks: np.ndarray,
                      vs: np.ndarray, scale: float, samples: Optional[Sequence[int]] = None):
    """Attention of each sample's single query token over [prefix ; own suffix].

    q [S][Hq][D]; kp, vp [Hkv][Lp][D]; ks, vs [S][Hkv][Ls][D].
    Returns (O [S][Hq][D], lse [S][Hq]); samples not listed hold NaN.
    """
    S, Hq, D = q.shape
    Hkv, Lp, _ = kp.shape
    Ls = ks.shape[2]
    G = Hq // Hkv
    O = np.full((S, Hq, D), np.nan)
    lse = np.full((S, Hq), np.nan)
    kp64, vp64 = _widen(kp), _widen(vp)
    for s in (range(S) if samples is None else samples):
        for kvh in range(Hkv):
            kcat = np.concatenate([kp64[kvh], _widen(ks[s, kvh])], axis=0)
            vcat = np.concatenate([vp64[kvh], _widen(vs[s, kvh])], axis=0)
            for h in range(kvh * G, (kvh + 1) * G):
                O[s, h], lse[s, h] = attend_row(q[s, h], kcat, vcat, scale)
    return O, lse


def attend_anchor_blocks(q: np.ndarray, ka: np.ndarray, va: np.ndarray, kb: np.ndarray,
                         vb: np.ndarray, scale: float, blocks: Optional[Sequence[int]] = None,
                         rows: Optional[Iterable[Tuple[int, int, int]]] = None):
    """Context encoding with an anchor block, per block of queries.

    q [N][Lb][Hq][D] (the queries of N context blocks); ka, va [Hkv][A][D]
    (the anchor block); kb, vb [N][Hkv][Lb][D] (each block's own keys and
    values).  Block b's query token i attends over [anchor ; block b] with
    every anchor key visible and the block's own keys t <= i.
    ``rows`` restricts the work to the listed (block, token, head) rows.
    Returns (O [N][Lb][Hq][D], lse [N][Lb][Hq]); rows not computed hold NaN.
    """
    N, Lb, Hq, D = q.shape
    Hkv, A, _ = ka.shape
    O = np.full((N, Lb, Hq, D), np.nan)
    lse = np.full((N, Lb, Hq), np.nan)
    want = {}
    if rows is not None:
        for (b, i, h) in rows:
            want.setdefault(b, []).append((0, i, h))
    for b in (range(N) if blocks is None else blocks) if rows is None else sorted(want):
        kc = np.concatenate([_widen(ka), _widen(kb[b])], axis=1)[None]  # [1][Hkv][A+Lb][D]
        vc = np.concatenate([_widen(va), _widen(vb[b])], axis=1)[None]
        Ob, lb = attend(q[b][None], kc, vc, [A + Lb], scale, causal=True, rows=want.get(b))
        O[b], lse[b] = Ob[0], lb[0]
    return O, lse


# ----------------------------------------------------------------------------
# Energy view
# ----------------------------------------------------------------------------
def energy(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
           zeta: Optional[np.ndarray] = None) -> float:
    """F(zeta) = ln sum_t exp(scale * q.k_t + zeta.v_t) for one query row."""
    q, k, v = _widen(q), _widen(k), _widen(v)
    if k.shape[0] == 0:
        return -math.inf
    x = scale * (k @ q)
    if zeta is not None:
        x = x + v @ np.asarray(zeta, dtype=np.float64)
    M = x.max()
    return M + math.log(np.exp(x - M).sum())


def energy_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, kv_lens, scale: float,
                zeta: np.ndarray, causal: bool = False,
                rows: Optional[Iterable[Tuple[int, int, int]]] = None) -> np.ndarray:
    """F(zeta) of every row of a decode call (or of the listed (b, i, h) rows),
    each over that row's visible keys; zeta has the shape of q, one auxiliary
    vector per row.  Returns float64 [B][q_len][Hq]; rows not listed hold NaN."""
    B, q_len, Hq, D = q.shape
    G = Hq // k.shape[1]
    lens = np.asarray(kv_lens, dtype=np.int64).reshape(B)
    out = np.full((B, q_len, Hq), np.nan)
    if rows is None:
        rows = [(b, i, h) for b in range(B) for i in range(q_len) for h in range(Hq)]
    for (b, i, h) in rows:
        n = visible(int(lens[b]), q_len, i, causal)
        out[b, i, h] = energy(q[b, i, h], k[b, h // G, :n], v[b, h // G, :n], scale,
                              _widen(zeta[b, i, h]))
    return out


# ----------------------------------------------------------------------------
# Chunk statistics and their merge
# ----------------------------------------------------------------------------
def chunk_partial(s: np.ndarray, v: np.ndarray):
    """(m, l, o) of one chunk: s[n] scaled logits, v[n, D] values."""
    s = np.asarray(s, dtype=np.float64)
    v = _widen(v)
    if s.size == 0 or not np.isfinite(s).any():
        return (-math.inf, 0.0, np.zeros(v.shape[1]))
    m = s.max()
    e = np.exp(s - m)
    return (m, e.sum(), e @ v)


def merge(a, b):
    """Combine two chunk records; (-inf, 0, 0) is the identity."""
    ma, la, oa = a
    mb, lb, ob = b
    m = max(ma, mb)
    if m == -math.inf:
        return (-math.inf, 0.0, np.zeros_like(oa))
    wa = math.exp(ma - m) if ma != -math.inf else 0.0
    wb = math.exp(mb - m) if mb != -math.inf else 0.0
    return (m, la * wa + lb * wb, oa * wa + ob * wb)


def finalize(p):
    """(O, lse) from a merged record: O = o / l, lse = m + ln l."""
    m, l, o = p
    if l == 0.0:
        return np.zeros_like(o), -math.inf
    return o / l, m + math.log(l)
