"""Energy at a given zeta on the GPU (through the C ABI).

F(zeta) = ln sum_t exp(scale q.k_t + zeta.v_t) per row is compared with the
oracle's fp64 value (lse bar), and the identity that makes the energy view
useful is checked on the device itself: central differences of F in zeta
reproduce the attention output O of attn_decode.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import O_TOL, check_rows, dev, say, workload_tensors
from long_context_exact_split_amd import binding, inputs

pytestmark = pytest.mark.gpu


def zeta_like(w, seed, scale=0.5):
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal(w.q.shape) * scale).astype(np.float32)
    return inputs.f32_to_bf16(z) if w.dtype == "bf16" else z


def widen(a):
    return inputs.bf16_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


ZETA = [
    # B, q_len, Hq, Hkv, D, L, dtype, causal, lens
    (1, 1, 1, 1, 64, 4096, "f32", False, None),
    (3, 1, 32, 8, 128, 2049, "bf16", False, [2049, 0, 1000]),
    (2, 1, 8, 8, 64, 3000, "bf16", False, [3000, 17]),
    (2, 4, 64, 8, 128, 1500, "bf16", True, [1500, 900]),  # R = 32 rows: still vector ALUs
    (2, 3, 6, 2, 128, 777, "f32", True, [777, 3]),
]


@pytest.mark.parametrize("case", ZETA, ids=[f"B{c[0]}_ql{c[1]}_Hq{c[2]}_Hkv{c[3]}_D{c[4]}_L{c[5]}_{c[6]}" for c in ZETA])
def test_energy_zeta_against_oracle(case):
    B, q_len, Hq, Hkv, D, L, dt, causal, lens = case
    w = inputs.make_decode("zeta", 700 + L, B=B, q_len=q_len, Hq=Hq, Hkv=Hkv, D=D, L_max=L,
                           kv_lens=lens, dtype=dt, causal=causal, nan_pad=True)
    z = zeta_like(w, L)
    q, k, v, lens_t = workload_tensors(w)
    F = binding.decode_energy_zeta(q, k, v, dev(z), lens_t, scale=w.scale, causal=causal)
    F0 = binding.decode_energy_zeta(q, k, v, dev(np.zeros_like(z)), lens_t, scale=w.scale,
                                    causal=causal)
    torch.cuda.synchronize()
    Fr = oracle.energy_rows(w.q, w.k, w.v, w.kv_lens, w.scale, widen(z), causal)
    check_rows(None, F.cpu().numpy(), None, Fr, what=f"F(zeta) {case}")
    _, lr = oracle.attend(w.q, w.k, w.v, w.kv_lens, w.scale, causal)
    check_rows(None, F0.cpu().numpy(), None, lr, what=f"F(0) = lse {case}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_zeta_gradient_is_the_attention_output(dt):
    """(F(h e_j) - F(-h e_j)) / 2h on the GPU against O_j from attn_decode, for
    every row and a spread of dimensions j; h = 2^-6 is exact in bf16."""
    w = inputs.make_decode("zeta_grad", 811, B=2, q_len=1, Hq=8, Hkv=2, D=128, L_max=3000,
                           kv_lens=[3000, 1200], dtype=dt)
    q, k, v, lens_t = workload_tensors(w)
    O, _ = binding.decode(q, k, v, lens_t, scale=w.scale)
    h = 2.0 ** -6
    worst = 0.0
    for j in (0, 1, 37, 64, 127):
        e = np.zeros(w.q.shape, np.float32)
        e[..., j] = h
        zp = inputs.f32_to_bf16(e) if dt == "bf16" else e
        zm = inputs.f32_to_bf16(-e) if dt == "bf16" else -e
        Fp = binding.decode_energy_zeta(q, k, v, dev(zp), lens_t, scale=w.scale)
        Fm = binding.decode_energy_zeta(q, k, v, dev(zm), lens_t, scale=w.scale)
        torch.cuda.synchronize()
        fd = ((Fp.double() - Fm.double()) / (2 * h)).cpu().numpy()
        err = np.abs(fd - O[..., j].double().cpu().numpy())
        worst = max(worst, float(err.max()))
        assert (err <= O_TOL).all(), f"dF/dzeta_{j} vs O_{j}: {err.max():.3e}"
    say(f"  central differences of F vs O ({dt}): max err {worst:.2e}")


def test_energy_zeta_full_size_8b_shape():
    """Llama-3-8B-shaped GQA decode (B=8, L=32768): F(zeta) on every row."""
    w = inputs.llama3_8b_gqa(seed=2)
    z = zeta_like(w, 3, scale=0.25)
    q, k, v, lens_t = workload_tensors(w)
    F = binding.decode_energy_zeta(q, k, v, dev(z), lens_t, scale=w.scale)
    torch.cuda.synchronize()
    Fr = oracle.energy_rows(w.q, w.k, w.v, w.kv_lens, w.scale, widen(z))
    check_rows(None, F.cpu().numpy(), None, Fr, what="F(zeta) 8B shape")
