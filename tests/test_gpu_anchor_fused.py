"""The anchor prefill's finalising path on the GPU.

For shapes where every segment of both parts is one piece, the local split
merges each row's two records itself and writes O and lse (no merge launch).
Each case checks that the path is taken, compares every row with the fp64
oracle, and compares with the unfused path (anchor split, local split,
merge) that the test build of the library runs on request: the same two records are merged by
the same rule in the same order, so the results agree to rounding of a
fused multiply-add.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import check_rows, dev, say
from long_context_exact_split_amd import binding, inputs

pytestmark = pytest.mark.gpu

CASES = [
    # N, Lb, Hq, Hkv, D, A
    (1, 9, 8, 2, 128, 100),     # 36 rows: two-wave workgroups, partial row block
    (1, 23, 16, 4, 128, 64),    # 92 rows: four-wave workgroups, partial row block
    (2, 40, 8, 2, 128, 50),     # 160 rows: eight waves, partial row block
    (2, 64, 32, 8, 128, 64),    # 256 rows: one full row block per KV head
    (1, 2048, 64, 8, 64, 512),  # head_dim 64, 64 row blocks per KV head
    (2, 1024, 64, 8, 128, 64),  # 8192 rows per KV head, short anchor
]


def anchor_desc(N, Lb, Hq, Hkv, D, A):
    d = binding.AttnAnchorDesc()
    d.num_blocks, d.block_len, d.num_q_heads, d.num_kv_heads, d.head_dim = N, Lb, Hq, Hkv, D
    d.anchor_len, d.scale, d.dtype = A, 1.0 / np.sqrt(D), 0
    return d


def make(N, Lb, Hq, Hkv, D, A, seed):
    rng = np.random.default_rng(seed)
    bits = lambda *s: inputs.f32_to_bf16(rng.standard_normal(s, dtype=np.float32))
    return (bits(N, Lb, Hq, D), bits(Hkv, A, D), bits(Hkv, A, D), bits(N, Hkv, Lb, D),
            bits(N, Hkv, Lb, D))


@pytest.mark.parametrize("case", CASES, ids=[f"N{c[0]}_Lb{c[1]}_Hq{c[2]}_Hkv{c[3]}_D{c[4]}_A{c[5]}" for c in CASES])
def test_fused_anchor_matches_oracle_and_unfused(case):
    N, Lb, Hq, Hkv, D, A = case
    say(f"fused anchor {case}")
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert binding.testing_anchor_fuses(anchor_desc(*case), cu), "shape no longer fuses"
    q, ka, va, kb, vb = make(*case, seed=Lb + 31 * A)
    t = [dev(x) for x in (q, ka, va, kb, vb)]
    scale = 1.0 / np.sqrt(D)
    O, lse = binding.prefill_anchor(*t, scale=scale)
    Ou, lseu = binding.testing_prefill_anchor_unfused(*t, scale=scale)
    torch.cuda.synchronize()
    O, lse, Ou, lseu = (x.cpu().numpy() for x in (O, lse, Ou, lseu))
    Or, lr = oracle.attend_anchor_blocks(q, ka, va, kb, vb, scale)
    check_rows(O, lse, Or, lr, what=f"fused anchor {case}")
    dO = float(np.abs(O - Ou).max())
    dl = float(np.abs(lse - lseu).max())
    say(f"  fused vs unfused: max|dO|={dO:.2e} max|dlse|={dl:.2e}")
    assert dO <= 1e-6 * max(1.0, float(np.abs(Ou).max())) and dl <= 1e-6 * max(1.0, float(np.abs(lseu).max()))
