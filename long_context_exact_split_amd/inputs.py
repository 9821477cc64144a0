"""Seeded synthetic workloads for exact split-KV attention decoding.

This module draws the inputs that both the CPU oracle and the HIP path consume:
Gaussian queries, keys and values, their rounding to bfloat16, ragged KV
lengths, planted "needle" keys, heavy-tailed key rows and NaN padding past each
sequence's end.  It contains none of the attention arithmetic (no logits, no
softmax, no merge), so it can serve both sides without coupling them.

Layouts (last axis contiguous):
  Q     [B][q_len][Hq][D]
  K, V  [B][Hkv][L_max][D]
  query head h reads KV head h // (Hq // Hkv)   (contiguous GQA groups)

bfloat16 tensors are carried as ``uint16`` bit patterns; ``bf16_to_f32`` turns
them back into exactly representable float32 values.

Random streams: numpy ``Generator(PCG64)``, one child ``SeedSequence`` per
role (Q, extras, and one per (batch, 64 Ki-token slab) of K/V), so that any slab
of a multi-GB cache can be regenerated on its own and generation runs in
parallel threads.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

SLAB_TOKENS = 65536
BF16_NAN = np.uint16(0x7FC0)


# ----------------------------------------------------------------------------
# bfloat16 bit handling
# ----------------------------------------------------------------------------
def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ----------------------------------------------------------------------------
# Workload containers
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    """One decode call's inputs.

    ``q``, ``k``, ``v`` hold uint16 bf16 bits when ``dtype == "bf16"`` and
    float32 values when ``dtype == "f32"``.  ``kv_lens[b]`` is the number of
    cached tokens of sequence b (for ``causal`` it includes the q_len new
    tokens, which sit at positions ``L_b - q_len .. L_b - 1``).
    """

    name: str
    seed: int
    dtype: str
    B: int
    q_len: int
    Hq: int
    Hkv: int
    D: int
    L_max: int
    kv_lens: np.ndarray
    scale: float
    causal: bool
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    chunk_len: int = 0
    notes: dict = dataclasses.field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def values(self, which: str) -> np.ndarray:
        """float32 view of q/k/v (exact for bf16 inputs)."""
        a = getattr(self, which)
        return bf16_to_f32(a) if self.dtype == "bf16" else a

    def kv_tokens(self) -> int:
        return int(np.asarray(self.kv_lens, dtype=np.int64).sum())


@dataclasses.dataclass
class BifurcatedWorkload:
    """Shared-prefix batch sampling: S samples share one prefix KV.

    Q [S][Hq][D]; Kp, Vp [Hkv][Lp][D]; Ks, Vs [S][Hkv][Ls][D]; all bf16 bits.
    """

    name: str
    seed: int
    S: int
    Hq: int
    Hkv: int
    D: int
    Lp: int
    Ls: int
    scale: float
    q: np.ndarray
    kp: np.ndarray
    vp: np.ndarray
    ks: np.ndarray
    vs: np.ndarray

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


# ----------------------------------------------------------------------------
# Draw helpers
# ----------------------------------------------------------------------------
def _normal_bits(rng: np.random.Generator, shape, as_bf16: bool) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bf16(x) if as_bf16 else x


def _fill_kv(children, k: np.ndarray, v: np.ndarray, L_max: int, as_bf16: bool,
             slab: int = SLAB_TOKENS) -> None:
    """Fill K and V [B][Hkv][L_max][D] slab by slab from per-slab child seeds."""
    B, Hkv, _, D = k.shape
    n_slabs = (L_max + slab - 1) // slab

    def job(idx):
        b, j = divmod(idx, n_slabs)
        t0, t1 = j * slab, min(L_max, (j + 1) * slab)
        rng = np.random.Generator(np.random.PCG64(children[idx]))
        k[b, :, t0:t1, :] = _normal_bits(rng, (Hkv, t1 - t0, D), as_bf16)
        v[b, :, t0:t1, :] = _normal_bits(rng, (Hkv, t1 - t0, D), as_bf16)

    todo = range(B * n_slabs)
    if B * n_slabs == 1:
        job(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(job, todo))


def _roots(seed: int, n_kv: int):
    ss = np.random.SeedSequence(seed)
    q_ss, extra_ss, kv_ss = ss.spawn(3)
    return q_ss, extra_ss, kv_ss.spawn(n_kv)


def make_decode(name: str, seed: int, *, B: int, q_len: int, Hq: int, Hkv: int, D: int,
                L_max: int, kv_lens=None, dtype: str = "bf16", causal: bool = False,
                scale: Optional[float] = None, chunk_len: int = 0,
                nan_pad: bool = False) -> Workload:
    """Gaussian N(0,1) Q/K/V for a dense or ragged decode call.

    ``kv_lens`` may be None (every sequence full), an int sequence, or the
    string "uniform:lo:hi" (integer lengths drawn uniformly, inclusive, from
    the extras stream).  With ``nan_pad`` every K/V token at or past L_b is a
    NaN, so that any read of padding poisons the result.
    """
    assert Hq % Hkv == 0
    as_bf16 = dtype == "bf16"
    n_slabs = max(1, (L_max + SLAB_TOKENS - 1) // SLAB_TOKENS)
    q_ss, extra_ss, kv_children = _roots(seed, B * n_slabs)
    q_rng = np.random.Generator(np.random.PCG64(q_ss))
    extra = np.random.Generator(np.random.PCG64(extra_ss))
    q = _normal_bits(q_rng, (B, q_len, Hq, D), as_bf16)
    et = np.uint16 if as_bf16 else np.float32
    k = np.empty((B, Hkv, L_max, D), dtype=et)
    v = np.empty((B, Hkv, L_max, D), dtype=et)
    _fill_kv(kv_children, k, v, L_max, as_bf16)
    if kv_lens is None:
        lens = np.full(B, L_max, dtype=np.int32)
    elif isinstance(kv_lens, str) and kv_lens.startswith("uniform:"):
        _, lo, hi = kv_lens.split(":")
        lens = extra.integers(int(lo), int(hi), endpoint=True, size=B).astype(np.int32)
    else:
        lens = np.asarray(kv_lens, dtype=np.int32).reshape(B)
    assert (lens >= 0).all() and (lens <= L_max).all()
    if nan_pad:
        pad = BF16_NAN if as_bf16 else np.float32(np.nan)
        for b in range(B):
            k[b, :, lens[b]:, :] = pad
            v[b, :, lens[b]:, :] = pad
    return Workload(name=name, seed=seed, dtype=dtype, B=B, q_len=q_len, Hq=Hq, Hkv=Hkv,
                    D=D, L_max=L_max, kv_lens=lens,
                    scale=(1.0 / math.sqrt(D)) if scale is None else float(scale),
                    causal=causal, q=q, k=k, v=v, chunk_len=chunk_len,
                    notes={"extra_rng": extra})


# ----------------------------------------------------------------------------
# The five workload shapes
# ----------------------------------------------------------------------------
def single_query_fp32(seed: int = 1) -> Workload:
    """Single-query decode: B=1, one head, d=64, L=4096, fp32, 8 chunks of 512."""
    w = make_decode("single_query_fp32", seed, B=1, q_len=1, Hq=1, Hkv=1, D=64, L_max=4096,
                    dtype="f32", chunk_len=512)
    w.notes.pop("extra_rng")
    return w


def llama3_8b_gqa(seed: int = 2, L: int = 32768, B: int = 8) -> Workload:
    """Llama-3-8B-shaped GQA decode: B=8, Hq=32, Hkv=8, d=128, L=32768, bf16."""
    w = make_decode("llama3_8b_gqa", seed, B=B, q_len=1, Hq=32, Hkv=8, D=128, L_max=L)
    w.notes.pop("extra_rng")
    return w


def plant_needles(w: Workload, logit: float = 30.0, literal_c: Optional[float] = None) -> None:
    """Plant one needle key per KV head (in place).

    Needle k* = c * q_hat, where q_hat is the unit vector of the group's first
    query head (h = G * kvh, token 0).  By default c = logit / (scale * |q|), so
    that head's scaled logit is ``logit`` before k* is rounded to bf16; with
    ``literal_c`` the constant c is used as is.  Positions are uniform in
    [0, L_b) from the extras stream; V rows are left unchanged.
    """
    extra: np.random.Generator = w.notes["extra_rng"]
    G = w.G
    qf = w.values("q").astype(np.float64)
    pos = []
    for b in range(w.B):
        for kvh in range(w.Hkv):
            n = int(extra.integers(0, int(w.kv_lens[b])))
            qv = qf[b, 0, G * kvh]
            nrm = float(np.sqrt(np.dot(qv, qv)))
            c = literal_c if literal_c is not None else logit / (w.scale * nrm)
            kstar = (c * qv / nrm).astype(np.float32)
            w.k[b, kvh, n, :] = f32_to_bf16(kstar) if w.dtype == "bf16" else kstar
            pos.append((b, kvh, n))
    w.notes["needles"] = pos


def long_context_gqa(L: int = 5_120_000, seed: int = 3, needle_logit: float = 30.0,
                     literal_c: Optional[float] = None) -> Workload:
    """Long-context GQA decode: B=1, Hq=32, Hkv=8, d=128, bf16, one needle per KV head."""
    w = make_decode("long_context_gqa", seed, B=1, q_len=1, Hq=32, Hkv=8, D=128, L_max=L)
    plant_needles(w, logit=needle_logit, literal_c=literal_c)
    w.notes.pop("extra_rng")
    return w


def llama31_70b_ragged(seed: int = 5, L_max: int = 131072, L_lo: int = 8192,
                       B: int = 16, heavy_frac: float = 0.01, heavy_mul: float = 8.0) -> Workload:
    """Llama-3.1-70B-shaped ragged decode: B=16, Hq=64, Hkv=8, d=128, 4 causal
    query tokens per sequence, lengths uniform in [8192, 131072], 1% of key rows
    multiplied by 8 (heavy-tailed logits), NaN padding past each length."""
    w = make_decode("llama31_70b_ragged", seed, B=B, q_len=4, Hq=64, Hkv=8, D=128,
                    L_max=L_max, kv_lens=f"uniform:{L_lo}:{L_max}", causal=True, nan_pad=True)
    extra: np.random.Generator = w.notes.pop("extra_rng")
    heavy = 0
    for b in range(w.B):
        n = int(w.kv_lens[b])
        mask = extra.random((w.Hkv, n)) < heavy_frac
        for kvh in range(w.Hkv):
            rows = np.nonzero(mask[kvh])[0]
            if rows.size:
                vals = bf16_to_f32(w.k[b, kvh, rows, :]) * np.float32(heavy_mul)
                w.k[b, kvh, rows, :] = f32_to_bf16(vals)
            heavy += rows.size
    w.notes["heavy_rows"] = heavy
    return w


def bifurcated_prefix(seed: int = 4, S: int = 64, Hq: int = 32, Hkv: int = 8, D: int = 128,
                      Lp: int = 16384, Ls: int = 512) -> BifurcatedWorkload:
    """Bifurcated shared-prefix sampling: 64 samples share a 16384-token prefix
    KV and each has its own 512-token decode KV; 32 query / 8 KV heads, d=128."""
    ss = np.random.SeedSequence(seed)
    sq, skp, sks = ss.spawn(3)
    q = _normal_bits(np.random.Generator(np.random.PCG64(sq)), (S, Hq, D), True)
    kp = np.empty((1, Hkv, Lp, D), np.uint16)
    vp = np.empty((1, Hkv, Lp, D), np.uint16)
    n_p = (Lp + SLAB_TOKENS - 1) // SLAB_TOKENS
    _fill_kv(skp.spawn(n_p), kp, vp, Lp, True)
    ks = np.empty((S, Hkv, Ls, D), np.uint16)
    vs = np.empty((S, Hkv, Ls, D), np.uint16)
    n_s = (Ls + SLAB_TOKENS - 1) // SLAB_TOKENS
    _fill_kv(sks.spawn(S * n_s), ks, vs, Ls, True)
    return BifurcatedWorkload(name="bifurcated_prefix", seed=seed, S=S, Hq=Hq, Hkv=Hkv, D=D,
                              Lp=Lp, Ls=Ls, scale=1.0 / math.sqrt(D), q=q, kp=kp[0], vp=vp[0],
                              ks=ks, vs=vs)


@dataclasses.dataclass
class AnchorWorkload:
    """Context encoding with an anchor block: N context blocks of Lb tokens,
    each processed behind an A-token anchor.  Q [N][Lb][Hq][D]; Ka, Va
    [Hkv][A][D]; Kb, Vb [N][Hkv][Lb][D]; bf16 bits."""

    name: str
    seed: int
    Hq: int
    Hkv: int
    D: int
    A: int
    scale: float
    q: np.ndarray
    ka: np.ndarray
    va: np.ndarray
    kb: np.ndarray
    vb: np.ndarray


def anchor_blocks(seed: int = 6, N: int = 2, Lb: int = 8192, A: int = 8192, Hq: int = 32,
                  Hkv: int = 8, D: int = 128) -> AnchorWorkload:
    """Anchor-block context encoding: N = 2 blocks of 8192 tokens behind an
    8192-token anchor, 32 query / 8 KV heads, d = 128, bf16 N(0,1)."""
    ss = np.random.SeedSequence(seed)
    streams = [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(5)]
    shapes = [(N, Lb, Hq, D), (Hkv, A, D), (Hkv, A, D), (N, Hkv, Lb, D), (N, Hkv, Lb, D)]
    q, ka, va, kb, vb = (_normal_bits(r, sh, True) for r, sh in zip(streams, shapes))
    return AnchorWorkload(name="anchor_prefill", seed=seed, Hq=Hq, Hkv=Hkv, D=D, A=A,
                          scale=1.0 / math.sqrt(D), q=q, ka=ka, va=va, kb=kb, vb=vb)


# ----------------------------------------------------------------------------
# Paged KV caches
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class PagedCache:
    """K and V of a decode call stored in fixed-size pages.

    ``k_pool`` / ``v_pool`` are flat element arrays (uint16 bf16 bits or
    float32) of ``num_pages * page_stride`` elements.  Logical page j of
    sequence b (tokens [j*P, (j+1)*P)) lives in physical page
    ``block_table[b, j]``; element (token t, KV head kvh, dim e) of that
    sequence sits at
    ``block_table[b, t // P] * page_stride + kvh * head_stride + (t % P) * token_stride + e``.
    Table entries past a sequence's last page are -1, and physical pages no
    sequence uses are filled with NaN: neither may ever be read.
    """

    k_pool: np.ndarray
    v_pool: np.ndarray
    block_table: np.ndarray  # int32 [B][pages_per_seq]
    page_size: int
    num_pages: int
    page_stride: int
    head_stride: int
    token_stride: int
    layout: str  # "head_major" ([page][Hkv][P][D]) or "token_major" ([page][P][Hkv][D])
    shared_pages: int = 0

    @property
    def pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])


def page_cache(w: Workload, page_size: int, layout: str = "head_major", seed: int = 0,
               spare_pages: int = 0, share_prefix_tokens: int = 0) -> PagedCache:
    """Scatter the (dense) cache of ``w`` into a pool of pages of ``page_size``
    tokens, in a seeded random physical order.

    With ``share_prefix_tokens`` = n > 0, every sequence first gets sequence
    0's first n tokens (``w.k`` / ``w.v`` are changed in place, so the dense
    arrays stay the logical cache), and the whole pages among them are stored
    once and referenced by every sequence's table.  ``spare_pages`` extra
    physical pages hold NaN.
    """
    assert layout in ("head_major", "token_major")
    P = int(page_size)
    assert P >= 1 and P & (P - 1) == 0, "page size must be a power of two"
    B, Hkv, L_max, D = w.k.shape
    lens = np.asarray(w.kv_lens, dtype=np.int64)
    n_share = 0
    if share_prefix_tokens:
        n = int(min(share_prefix_tokens, lens.min()))
        for b in range(1, B):
            w.k[b, :, :n] = w.k[0, :, :n]
            w.v[b, :, :n] = w.v[0, :, :n]
        n_share = n // P  # whole pages only
    pages_per_seq = max(1, (L_max + P - 1) // P)
    used = [int((L + P - 1) // P) for L in lens]
    # Physical pages: the shared ones once, then every sequence's own pages.
    logical = [(0, j) for j in range(min(n_share, used[0]))]
    for b in range(B):
        logical += [(b, j) for j in range(n_share if b > 0 else min(n_share, used[0]), used[b])]
    num_pages = len(logical) + int(spare_pages)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, P, num_pages])))
    phys = rng.permutation(num_pages)[:len(logical)]
    table = np.full((B, pages_per_seq), -1, dtype=np.int32)
    for (b, j), p in zip(logical, phys):
        table[b, j] = p
        if b == 0 and j < n_share:
            table[1:, j] = p
    shape = (num_pages, Hkv, P, D) if layout == "head_major" else (num_pages, P, Hkv, D)
    nan = BF16_NAN if w.k.dtype == np.uint16 else np.float32(np.nan)
    pools = []
    for src in (w.k, w.v):
        pool = np.full(shape, nan, dtype=src.dtype)
        for (b, j), p in zip(logical, phys):
            t0 = j * P
            t1 = min(int(lens[b]), t0 + P)
            blk = src[b, :, t0:t1, :]                      # [Hkv][n][D]
            if layout == "head_major":
                pool[p, :, :t1 - t0, :] = blk
            else:
                pool[p, :t1 - t0, :, :] = blk.transpose(1, 0, 2)
        pools.append(pool.reshape(-1))
    if layout == "head_major":
        strides = (Hkv * P * D, P * D, D)
    else:
        strides = (P * Hkv * D, D, Hkv * D)
    return PagedCache(k_pool=pools[0], v_pool=pools[1], block_table=table, page_size=P,
                      num_pages=num_pages, page_stride=strides[0], head_stride=strides[1],
                      token_stride=strides[2], layout=layout, shared_pages=n_share)
