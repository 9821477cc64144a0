"""Seeded random shapes through the C ABI against the fp64 oracle, every row.

The shapes are drawn once from a fixed seed, so each case has a stable name
and a failure can be rerun alone.  They cover the three split kernels and
both merges at once: batch sizes, query blocks (causal or not, up to several
row blocks of the shared-tile kernel, GQA ratios that do and do not divide a
row block), head sizes, element types, ragged and empty sequences, forced
chunk lengths, paged pools of several page sizes and both layouts, and
energy-only calls; and random bifurcated batches (empty prefix or suffix
included) and anchor-block prefills (empty anchor included).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import check_rows, dev, say, workload_tensors
from long_context_exact_split_amd import binding, inputs

pytestmark = pytest.mark.gpu


def _cases(n=120, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        prefill = k % 3 == 2  # a query block of 40-200 tokens: several row blocks when causal
        dt = "f32" if (not prefill and rng.random() < 0.2) else "bf16"
        B = int(rng.integers(1, 3 if prefill else 5))
        Hkv = int(rng.integers(1, 3 if prefill else 5))
        G = int(rng.integers(1, 10))
        q_len = (int(rng.integers(40, 201)) if prefill
                 else int(rng.choice([1, 1, 2, 4, int(rng.integers(5, 70))])))
        D = int(rng.choice([64, 128]))
        L = int(rng.integers(1, 1500))
        causal = bool(q_len > 1 and (prefill or rng.random() < 0.8))
        lens = [int(x) for x in rng.integers(0, L + 1, size=B)] if rng.random() < 0.6 else None
        chunk = int(64 * rng.integers(1, 9)) if (not prefill and rng.random() < 0.2) else 0
        paged = None
        if chunk == 0 and rng.random() < 0.3:
            paged = (int(rng.choice([1, 4, 16, 64])), str(rng.choice(["head_major", "token_major"])))
        energy = bool(rng.random() < 0.25)
        out.append((k, dt, B, Hkv, G, q_len, D, L, causal, lens, chunk, paged, energy))
    return out


CASES = _cases()


def _id(c):
    k, dt, B, Hkv, G, q_len, D, L, causal, lens, chunk, paged, energy = c
    return (f"{k:02d}_{dt}_B{B}_Hkv{Hkv}_G{G}_ql{q_len}_D{D}_L{L}" + ("_causal" if causal else "")
            + ("_ragged" if lens else "") + (f"_C{chunk}" if chunk else "")
            + (f"_P{paged[0]}{paged[1][0]}" if paged else "") + ("_energy" if energy else ""))


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_shape(case):
    k, dt, B, Hkv, G, q_len, D, L, causal, lens, chunk, paged, energy = case
    say(f"random shape {_id(case)}")
    w = inputs.make_decode("random", 3000 + k, B=B, q_len=q_len, Hq=G * Hkv, Hkv=Hkv, D=D,
                           L_max=L, kv_lens=lens, dtype=dt, causal=causal, nan_pad=True)
    q, kk, v, lens_t = workload_tensors(w)
    if paged is not None:
        P, layout = paged
        pc = inputs.page_cache(w, P, layout=layout, seed=k, spare_pages=1)
        shape = (pc.num_pages, Hkv, P, D) if layout == "head_major" else (pc.num_pages, P, Hkv, D)
        cache = binding.PagedCache(dev(pc.k_pool.reshape(shape)), dev(pc.v_pool.reshape(shape)),
                                   torch.from_numpy(pc.block_table).cuda(), layout=layout,
                                   max_kv_len=L)
        lens_p = torch.from_numpy(w.kv_lens.astype(np.int32)).cuda()
        if energy:
            lse = binding.decode_energy_paged(q, cache, lens_p, scale=w.scale, causal=causal)
            O = None
        else:
            O, lse = binding.decode_paged(q, cache, lens_p, scale=w.scale, causal=causal)
    elif energy:
        lse = binding.decode_energy(q, kk, lens_t, scale=w.scale, causal=causal, chunk_len=chunk)
        O = None
    else:
        O, lse = binding.decode(q, kk, v, lens_t, scale=w.scale, causal=causal, chunk_len=chunk)
    torch.cuda.synchronize()
    Or, lr = oracle.attend(w.q, w.k, None if energy else w.v, w.kv_lens, w.scale, causal)
    check_rows(None if O is None else O.cpu().numpy(), lse.cpu().numpy(), Or, lr,
               what=f"random {_id(case)}")


def _bif_cases(n=24, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        Hkv = int(rng.integers(1, 5))
        G = int(rng.integers(1, 10))
        out.append((k, int(rng.integers(1, 80)), G * Hkv, Hkv, int(rng.choice([64, 128])),
                    int(rng.integers(0, 3000)), int(rng.integers(0, 700))))
    return out


BIF = _bif_cases()


@pytest.mark.parametrize("case", BIF, ids=[f"{c[0]:02d}_S{c[1]}_Hq{c[2]}_Hkv{c[3]}_D{c[4]}_Lp{c[5]}_Ls{c[6]}" for c in BIF])
def test_random_bifurcated(case):
    k, S, Hq, Hkv, D, Lp, Ls = case
    say(f"random bifurcated {case}")
    w = inputs.bifurcated_prefix(seed=500 + k, S=S, Hq=Hq, Hkv=Hkv, D=D, Lp=Lp, Ls=Ls)
    O, lse = binding.decode_bifurcated(*[dev(x) for x in (w.q, w.kp, w.vp, w.ks, w.vs)],
                                       scale=w.scale)
    torch.cuda.synchronize()
    Or, lr = oracle.attend_bifurcated(w.q, w.kp, w.vp, w.ks, w.vs, w.scale)
    check_rows(O.cpu().numpy()[:, None], lse.cpu().numpy()[:, None], Or[:, None], lr[:, None],
               what=f"random bifurcated {case}")


def _anchor_cases(n=24, seed=99):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        Hkv = int(rng.integers(1, 4))
        G = int(rng.integers(1, 9))
        out.append((k, int(rng.integers(1, 4)), int(rng.integers(1, 260)), G * Hkv, Hkv,
                    int(rng.choice([64, 128])), int(rng.integers(0, 1200))))
    return out


ANCHOR = _anchor_cases()


@pytest.mark.parametrize("case", ANCHOR, ids=[f"{c[0]:02d}_N{c[1]}_Lb{c[2]}_Hq{c[3]}_Hkv{c[4]}_D{c[5]}_A{c[6]}" for c in ANCHOR])
def test_random_anchor_blocks(case):
    k, N, Lb, Hq, Hkv, D, A = case
    say(f"random anchor {case}")
    rng = np.random.default_rng(900 + k)
    bits = lambda *s: inputs.f32_to_bf16(rng.standard_normal(s, dtype=np.float32))
    q, ka, va, kb, vb = (bits(N, Lb, Hq, D), bits(Hkv, A, D), bits(Hkv, A, D),
                         bits(N, Hkv, Lb, D), bits(N, Hkv, Lb, D))
    scale = 1.0 / np.sqrt(D)
    O, lse = binding.prefill_anchor(dev(q), dev(ka), dev(va), dev(kb), dev(vb), scale=scale)
    torch.cuda.synchronize()
    Or, lr = oracle.attend_anchor_blocks(q, ka, va, kb, vb, scale)
    check_rows(O.cpu().numpy(), lse.cpu().numpy(), Or, lr, what=f"random anchor {case}")
