"""HIP path (through the C ABI) against the fp64 oracle, element by element.

Small shapes are compared on every output; the full-size workloads are
compared on every row the oracle can afford (all rows for the 8B-shaped GQA
decode and the bifurcated batch; sampled KV-head groups for the 5.12M-token
cache and the 70B-shaped ragged batch)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import check_rows, dev, say, workload_tensors
from long_context_exact_split_amd import binding, inputs

pytestmark = pytest.mark.gpu


def run_decode(w, chunk_len=None):
    q, k, v, lens = workload_tensors(w)
    O, lse = binding.decode(q, k, v, lens, scale=w.scale, causal=w.causal,
                            chunk_len=w.chunk_len if chunk_len is None else chunk_len)
    torch.cuda.synchronize()
    return O.cpu().numpy(), lse.cpu().numpy()


def oracle_decode(w, rows=None):
    return oracle.attend(w.q, w.k, w.v, w.kv_lens, w.scale, w.causal, rows=rows)


def oracle_decode_parallel(w, rows, energy_only=False):
    """The oracle on sampled rows of a long cache: one call per (sequence, KV
    head) group, the groups in parallel host threads (numpy releases the
    interpreter in its kernels), each printing when it is done."""
    from concurrent.futures import ThreadPoolExecutor
    groups = {}
    for r in rows:
        groups.setdefault((r[0], r[2] // w.G), []).append(r)

    def one(g):
        out = oracle.attend(w.q, w.k, None if energy_only else w.v, w.kv_lens, w.scale,
                            w.causal, rows=g)
        say(f"  oracle group (b, kvh) = ({g[0][0]}, {g[0][2] // w.G}) done")
        return g, out
    with ThreadPoolExecutor(min(8, len(groups))) as ex:
        parts = list(ex.map(one, groups.values()))
    O = None if energy_only else np.full(w.q.shape, np.nan)
    lse = np.full(w.q.shape[:3], np.nan)
    for g, (Og, lg) in parts:
        for r in g:
            lse[r] = lg[r]
            if O is not None:
                O[r] = Og[r]
    return O, lse


# ----------------------------------------------------------------------------
# The five workload shapes
# ----------------------------------------------------------------------------
def test_single_query_fp32_eight_chunks():
    w = inputs.single_query_fp32(seed=1)
    desc = binding.make_desc(batch=1, q_len=1, num_q_heads=1, num_kv_heads=1, head_dim=64,
                             max_kv_len=4096, chunk_len=512, dtype=binding.ATTN_F32)
    p = binding.plan(desc)
    assert p["chunks_per_seq"] == 8
    say(f"single_query_fp32 plan: {p}")
    O, lse = run_decode(w)
    Or, lr = oracle_decode(w)
    check_rows(O, lse, Or, lr, what="single_query_fp32")


def test_llama3_8b_gqa_full():
    w = inputs.llama3_8b_gqa(seed=2)
    O, lse = run_decode(w)
    Or, lr = oracle_decode(w)
    check_rows(O, lse, Or, lr, what="llama3_8b_gqa (B=8, L=32768)")


# ----------------------------------------------------------------------------
# Small shapes spanning several tiles and a ragged tail
# ----------------------------------------------------------------------------
SMALL = [
    # B, q_len, Hq, Hkv, D, L, dtype, causal, lens
    (1, 1, 1, 1, 64, 4096, "f32", False, None),
    (1, 1, 8, 8, 128, 1000, "f32", False, None),
    (2, 1, 4, 2, 128, 777, "f32", False, [777, 300]),
    (3, 1, 32, 8, 128, 2049, "bf16", False, None),
    (2, 1, 8, 8, 64, 5000, "bf16", False, [5000, 4097]),
    (2, 1, 16, 2, 128, 3000, "bf16", False, [1, 2999]),
    (2, 1, 6, 2, 64, 1500, "bf16", False, [1500, 17]),
    (4, 1, 10, 2, 128, 1234, "bf16", False, "uniform:1:1234"),
    (2, 4, 8, 2, 128, 2000, "bf16", True, [2000, 1003]),
    (2, 2, 4, 4, 64, 333, "bf16", True, [333, 2]),
    (3, 3, 2, 1, 128, 700, "f32", True, [700, 3, 1]),
    (2, 4, 64, 8, 128, 4500, "bf16", True, [4500, 4096]),
    (1, 4, 32, 8, 64, 999, "bf16", True, None),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}_ql{c[1]}_Hq{c[2]}_Hkv{c[3]}_D{c[4]}_L{c[5]}_{c[6]}{'_causal' if c[7] else ''}" for c in SMALL])
def test_small_shapes(case):
    B, q_len, Hq, Hkv, D, L, dt, causal, lens = case
    w = inputs.make_decode("small", 100 + L, B=B, q_len=q_len, Hq=Hq, Hkv=Hkv, D=D, L_max=L,
                           kv_lens=lens, dtype=dt, causal=causal, nan_pad=True)
    O, lse = run_decode(w)
    Or, lr = oracle_decode(w)
    check_rows(O, lse, Or, lr, what=f"small {case}")


# Dense query blocks (R = G * q_len > 8, bf16) run on the MFMA kernel.
MFMA = [
    # B, q_len, Hq, Hkv, D, L, causal, lens
    (2, 4, 64, 8, 128, 4500, True, [4500, 4096]),
    (1, 2, 8, 1, 128, 3000, True, None),
    (3, 3, 4, 1, 64, 777, True, [777, 3, 100]),
    (2, 1, 16, 1, 128, 2049, False, [2049, 31]),
    (1, 8, 64, 8, 128, 1500, True, None),        # R = 64: two row blocks
    (2, 5, 14, 2, 64, 1100, True, [1100, 600]),   # R = 35: padded second block
    (1, 4, 16, 2, 128, 40000, True, None),
    (2, 6, 16, 1, 128, 3000, True, [3000, 1000]),  # R = 96: shared-tile kernel, 4 waves
    (1, 8, 25, 1, 64, 2500, True, None),           # R = 200: 8 waves, padded rows
    (1, 4, 64, 1, 64, 1800, True, None),           # R = 256, D = 64
    (1, 1, 256, 1, 128, 5000, False, None),        # R = 256: a shared-prefix shape
]


def G_q(case):
    return case[2] // case[3] * case[1]


@pytest.mark.parametrize("case", MFMA, ids=[f"B{c[0]}_ql{c[1]}_Hq{c[2]}_Hkv{c[3]}_D{c[4]}_L{c[5]}" for c in MFMA])
def test_mfma_query_blocks(case):
    B, q_len, Hq, Hkv, D, L, causal, lens = case
    w = inputs.make_decode("mfma", 300 + L, B=B, q_len=q_len, Hq=Hq, Hkv=Hkv, D=D, L_max=L,
                           kv_lens=lens, causal=causal, nan_pad=True)
    desc = binding.make_desc(batch=B, q_len=q_len, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                             max_kv_len=L, causal=causal)
    assert binding.plan(desc)["kernel"] == (1 if G_q(case) <= 32 else 2)
    O, lse = run_decode(w)
    Or, lr = oracle_decode(w)
    check_rows(O, lse, Or, lr, what=f"mfma {case}")
    q, k, v, lens_t = workload_tensors(w)
    lse_e = binding.decode_energy(q, k, lens_t, causal=causal)
    torch.cuda.synchronize()
    check_rows(None, lse_e.cpu().numpy(), None, lr, what=f"mfma energy {case}")


@pytest.mark.parametrize("chunk_len", [64, 128, 512, 4096])
def test_forced_chunk_lengths(chunk_len):
    w = inputs.make_decode("chunks", 7, B=2, q_len=1, Hq=8, Hkv=2, D=128, L_max=3000,
                           kv_lens=[3000, 1700], nan_pad=True)
    O, lse = run_decode(w, chunk_len=chunk_len)
    Or, lr = oracle_decode(w)
    check_rows(O, lse, Or, lr, what=f"chunk_len={chunk_len}")


# ----------------------------------------------------------------------------
# Degenerate cases
# ----------------------------------------------------------------------------
def test_empty_cache_and_empty_rows():
    w = inputs.make_decode("empty", 3, B=3, q_len=2, Hq=4, Hkv=2, D=64, L_max=300,
                           kv_lens=[0, 1, 300], causal=True, nan_pad=True)
    O, lse = run_decode(w)
    Or, lr = oracle_decode(w)
    assert np.isneginf(lr[0]).all() and np.isneginf(lr[1, 0]).all()  # rows that see nothing
    check_rows(O, lse, Or, lr, what="empty rows")


def test_zero_length_cache():
    q = torch.randn(2, 1, 4, 128, device="cuda").to(torch.bfloat16)
    k = torch.empty(2, 2, 0, 128, device="cuda", dtype=torch.bfloat16)
    O, lse = binding.decode(q, k, k)
    torch.cuda.synchronize()
    assert torch.isneginf(lse).all() and (O == 0).all()
    lse_e = binding.decode_energy(q, k)
    torch.cuda.synchronize()
    assert torch.isneginf(lse_e).all()


def test_single_key_returns_its_value_row():
    w = inputs.make_decode("one", 5, B=1, q_len=1, Hq=4, Hkv=1, D=128, L_max=1)
    O, lse = run_decode(w)
    v = w.values("v")[0, 0, 0]
    assert np.abs(O[0, 0] - v[None, :]).max() <= 1e-6
    Or, lr = oracle_decode(w)
    check_rows(O, lse, Or, lr, what="single key")


def test_identical_keys_give_mean_of_v():
    w = inputs.make_decode("same", 6, B=1, q_len=1, Hq=2, Hkv=1, D=64, L_max=1000)
    w.k[0, 0, :] = w.k[0, 0, 0]
    O, lse = run_decode(w)
    mean_v = w.values("v")[0, 0].astype(np.float64).mean(axis=0)
    assert np.abs(O[0, 0] - mean_v[None]).max() <= 2e-3
    Or, lr = oracle_decode(w)
    check_rows(O, lse, Or, lr, what="identical keys")


CAUSAL_BLOCKS = [
    # B, q_len, Hq, Hkv, D, L, dtype, lens: causal calls over several row blocks
    (1, 96, 8, 2, 128, 700, "bf16", None),         # 384 rows: two blocks of 256
    (2, 300, 4, 1, 128, 1000, "bf16", [200, 1000]),  # q_len > L_b: early blocks see nothing
    (2, 7, 6, 2, 128, 500, "f32", [500, 5]),      # vector ALUs, 3 blocks of 8 rows
    (3, 40, 16, 2, 64, 333, "bf16", [333, 0, 41]),   # 320 rows, an empty sequence
]


@pytest.mark.parametrize("case", CAUSAL_BLOCKS, ids=[f"B{c[0]}_ql{c[1]}_Hq{c[2]}_Hkv{c[3]}_D{c[4]}_L{c[5]}_{c[6]}" for c in CAUSAL_BLOCKS])
def test_causal_query_blocks_over_several_row_blocks(case):
    """Each row block of a causal call is given only the keys its rows can
    see; every row still matches the oracle, and rows that see no key give
    lse = -inf and O = 0."""
    B, q_len, Hq, Hkv, D, L, dt, lens = case
    say(f"causal row blocks {case}")
    w = inputs.make_decode("causal_blocks", 900 + L, B=B, q_len=q_len, Hq=Hq, Hkv=Hkv, D=D,
                           L_max=L, kv_lens=lens, dtype=dt, causal=True, nan_pad=True)
    desc = binding.make_desc(batch=B, q_len=q_len, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                             max_kv_len=L, causal=True,
                             dtype=binding.ATTN_BF16 if dt == "bf16" else binding.ATTN_F32)
    assert binding.plan(desc, 256)["row_blocks"] > 1
    O, lse = run_decode(w)
    Or, lr = oracle_decode(w)
    check_rows(O, lse, Or, lr, what=f"causal row blocks {case}")
    q, k, v, lens_t = workload_tensors(w)
    lse_e = binding.decode_energy(q, k, lens_t, causal=True)
    torch.cuda.synchronize()
    check_rows(None, lse_e.cpu().numpy(), None, lr, what=f"causal row blocks energy {case}")


TWO_PHASE = [
    # B, q_len, Hq, Hkv, D, L, causal, lens, energy
    (2, 1, 32, 8, 128, 3000, False, [3000, 1234], False),   # vector ALUs
    (2, 4, 64, 8, 128, 4500, True, [4500, 4096], False),    # 32-row matrix-core kernel
    (1, 96, 8, 2, 128, 700, True, None, False),             # shared-tile, causal row blocks
    (2, 130, 16, 4, 64, 900, True, [900, 300], True),       # the same, energy only
]


@pytest.mark.parametrize("case", TWO_PHASE, ids=[f"B{c[0]}_ql{c[1]}_Hq{c[2]}_Hkv{c[3]}_D{c[4]}{'_energy' if c[8] else ''}" for c in TWO_PHASE])
def test_two_phases_give_the_one_call_result(case):
    """attn_decode_partials then attn_decode_merge (each planning the call by
    itself) reproduce attn_decode / attn_decode_energy bit for bit."""
    B, q_len, Hq, Hkv, D, L, causal, lens, energy = case
    w = inputs.make_decode("phases", 950 + L, B=B, q_len=q_len, Hq=Hq, Hkv=Hkv, D=D, L_max=L,
                           kv_lens=lens, causal=causal, nan_pad=True)
    q, k, v, lens_t = workload_tensors(w)
    ph = binding.Phases(q, k, None if energy else v, lens_t, scale=w.scale, causal=causal)
    ph.partials()
    ph.merge()
    if energy:
        lse1 = binding.decode_energy(q, k, lens_t, scale=w.scale, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(ph.lse, lse1)
    else:
        O1, lse1 = binding.decode(q, k, v, lens_t, scale=w.scale, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(ph.out, O1) and torch.equal(ph.lse, lse1)
    _, lr = oracle.attend(w.q, w.k, None, w.kv_lens, w.scale, causal)
    check_rows(None, ph.lse.cpu().numpy(), None, lr, what=f"two phases {case}")


def test_too_small_workspace_is_refused_and_nothing_is_written():
    """A workspace below the size query's answer: ATTN_ERR_WORKSPACE, and the
    outputs keep their contents (nothing was launched)."""
    import ctypes
    lib = binding.load_library()
    w = inputs.make_decode("ws", 12, B=2, q_len=1, Hq=8, Hkv=2, D=128, L_max=3000)
    q, k, v, _ = workload_tensors(w)
    d = binding.make_desc(batch=2, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                          max_kv_len=3000, scale=w.scale)
    need = binding.workspace_bytes(d)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    O = torch.full((2, 1, 8, 128), 7.0, device="cuda")
    lse = torch.full((2, 1, 8), 7.0, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.attn_decode(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(), O.data_ptr(),
                         lse.data_ptr(), ws.data_ptr(), need - 1, stream)
    torch.cuda.synchronize()
    assert binding.STATUS[st] == "ATTN_ERR_WORKSPACE"
    assert (O == 7.0).all() and (lse == 7.0).all()
    wb = inputs.bifurcated_prefix(seed=46, S=4, Lp=300, Ls=40)
    tb = [dev(x) for x in (wb.q, wb.kp, wb.vp, wb.ks, wb.vs)]
    bd = binding.bifurcated_desc(tb[0], tb[1], tb[3], wb.scale)
    n = ctypes.c_size_t(0)
    assert lib.attn_bifurcated_workspace_bytes(ctypes.byref(bd), ctypes.byref(n)) == 0 and n.value > 0
    wsb = torch.empty(n.value, dtype=torch.uint8, device="cuda")
    Ob = torch.full((4, wb.Hq, wb.D), 7.0, device="cuda")
    lseb = torch.full((4, wb.Hq), 7.0, device="cuda")
    st = lib.attn_decode_bifurcated(ctypes.byref(bd), *[t.data_ptr() for t in tb], Ob.data_ptr(),
                                    lseb.data_ptr(), wsb.data_ptr(), n.value - 1, stream)
    torch.cuda.synchronize()
    assert binding.STATUS[st] == "ATTN_ERR_WORKSPACE"
    assert (Ob == 7.0).all() and (lseb == 7.0).all()


def test_huge_logits_are_stable():
    w = inputs.make_decode("huge", 8, B=1, q_len=1, Hq=4, Hkv=1, D=128, L_max=4000, dtype="f32")
    w.q *= np.float32(40.0)  # logits of several hundred
    O, lse = run_decode(w)
    Or, lr = oracle_decode(w)
    assert np.abs(lr).max() > 100  # logits ~ N(0, 40^2): the max over 4000 keys is ~140
    check_rows(O, lse, Or, lr, what="huge logits")


SPIKES = [
    # B, q_len, Hq, Hkv, causal: vector-ALU rows, matrix-core kernel 1, shared-tile kernel 2
    (2, 1, 8, 2, False),
    (1, 4, 32, 4, True),
    (1, 6, 16, 1, True),
]


@pytest.mark.parametrize("case", SPIKES, ids=[f"B{c[0]}_ql{c[1]}_Hq{c[2]}_Hkv{c[3]}" for c in SPIKES])
def test_isolated_huge_logits_at_every_lane_position(case):
    """One key per 65-token stride aimed at one row with a logit of 200 + j
    (natural units, j = 0..63), so that across the cache the dominating key
    sits at every position modulo 64: whichever lanes or key slots hold it,
    every partial maximum that combines with it must see it, or its
    exponential overflows (2^288 and more)."""
    B, q_len, Hq, Hkv, causal = case
    L = 4500
    w = inputs.make_decode("spikes", 41 + Hq, B=B, q_len=q_len, Hq=Hq, Hkv=Hkv, D=128,
                           L_max=L, causal=causal)
    qf = w.values("q").astype(np.float64)
    G = Hq // Hkv
    for b in range(B):
        for kvh in range(Hkv):
            for j in range(64):
                i, h = j % q_len, kvh * G + (j // q_len) % G
                qv = qf[b, i, h]
                c = (200.0 + j) / (w.scale * float(np.dot(qv, qv)))
                w.k[b, kvh, 65 * j, :] = inputs.f32_to_bf16((c * qv).astype(np.float32))
    O, lse = run_decode(w)
    Or, lr = oracle_decode(w)
    assert lr.max() > 200
    check_rows(O, lse, Or, lr, what=f"spikes {case}")
    q, k, v, lens_t = workload_tensors(w)
    lse_e = binding.decode_energy(q, k, lens_t, causal=causal)
    torch.cuda.synchronize()
    check_rows(None, lse_e.cpu().numpy(), None, lr, what=f"spikes energy {case}")


# ----------------------------------------------------------------------------
# Properties of the path
# ----------------------------------------------------------------------------
FEW_TOKENS = [([5], 4, 1), ([1, 0, 2], 4, 1), ([3, 7], 32, 1), ([5], 16, 2), ([2, 9, 0, 4], 4, 1)]


@pytest.mark.parametrize("case", FEW_TOKENS, ids=[f"lens{c[0]}_Hq{c[1]}_ql{c[2]}" for c in FEW_TOKENS])
def test_ragged_lengths_below_the_planned_workgroups(case):
    """Lengths far below max_kv_len: the cached tokens (read on the device)
    come to fewer units than the workgroups the plan sized for max_kv_len, so
    only as many workgroups as units take a share.  The workspace is filled
    with NaN first: a record the merge read without a piece having written it
    would poison its row.  Decode and energy-only, vector-ALU and matrix-core
    kernels."""
    lens, Hq, q_len = case
    B = len(lens)
    w = inputs.make_decode("few_tokens", 61 + B, B=B, q_len=q_len, Hq=Hq, Hkv=1, D=128,
                           L_max=4096, kv_lens=lens, nan_pad=True)
    q, k, v, _ = workload_tensors(w)
    kv = torch.from_numpy(w.kv_lens.astype(np.int32)).cuda()
    ws = torch.full((4 << 20,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)
    O, lse = binding.decode(q, k, v, kv, scale=w.scale, workspace=ws)
    ws.view(torch.float32).fill_(float("nan"))
    lse_e = binding.decode_energy(q, k, kv, scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    Or, lr = oracle_decode(w)
    check_rows(O.cpu().numpy(), lse.cpu().numpy(), Or, lr, what=f"few tokens {case}")
    check_rows(None, lse_e.cpu().numpy(), None, lr, what=f"few tokens energy {case}")


def test_energy_lse_matches_decode_lse():
    w = inputs.make_decode("energy", 9, B=2, q_len=2, Hq=16, Hkv=4, D=128, L_max=5000,
                           kv_lens=[5000, 2222], causal=True, nan_pad=True)
    q, k, v, lens = workload_tensors(w)
    O, lse = binding.decode(q, k, v, lens, causal=True)
    lse_e = binding.decode_energy(q, k, lens, causal=True)
    torch.cuda.synchronize()
    _, lr = oracle.attend(w.q, w.k, None, w.kv_lens, w.scale, True)
    check_rows(None, lse_e.cpu().numpy(), None, lr, what="energy-only lse")
    assert torch.equal(lse_e, lse), "energy-only lse differs from attn_decode's lse"


def test_two_runs_bitwise_identical():
    w = inputs.make_decode("det", 10, B=2, q_len=1, Hq=32, Hkv=8, D=128, L_max=20000)
    q, k, v, lens = workload_tensors(w)
    O1, l1 = binding.decode(q, k, v, lens)
    O2, l2 = binding.decode(q, k, v, lens)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(l1, l2)


def test_chunking_does_not_change_the_result_beyond_rounding():
    w = inputs.make_decode("assoc", 11, B=1, q_len=1, Hq=8, Hkv=2, D=128, L_max=8192)
    a = run_decode(w, chunk_len=64)
    b = run_decode(w, chunk_len=8192)
    assert np.abs(a[0] - b[0]).max() < 1e-4 and np.abs(a[1] - b[1]).max() < 1e-5


# ----------------------------------------------------------------------------
# Full-size long-context and ragged workloads (sampled rows)
# ----------------------------------------------------------------------------
def _needle_rows(w, extra_heads=(5, 18, 27)):
    rows = [(0, 0, w.G * kvh) for (_, kvh, _) in w.notes["needles"]]
    return rows + [(0, 0, h) for h in extra_heads]


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_long_context_1m_needle():
    """The headline shape: decode, energy only and F(zeta) on one 1M-token
    cache, each against the oracle on the needle rows and three others; the
    energy-only lse equals the decode lse bit for bit on every row."""
    w = inputs.long_context_gqa(L=1 << 20, seed=31)
    say("generated 1M-token cache")
    q, k, v, lens = workload_tensors(w)
    O, lse = binding.decode(q, k, v, lens, scale=w.scale)
    lse_e = binding.decode_energy(q, k, lens, scale=w.scale)
    zrng = np.random.default_rng(17)
    zeta = inputs.f32_to_bf16(zrng.standard_normal(w.q.shape, dtype=np.float32) * np.float32(0.25))
    F = binding.decode_energy_zeta(q, k, v, dev(zeta), lens, scale=w.scale)
    torch.cuda.synchronize()
    O, lse, lse_e, F = (x.cpu().numpy() for x in (O, lse, lse_e, F))
    del q, k, v
    torch.cuda.empty_cache()
    assert np.array_equal(lse_e, lse), "energy-only lse differs from the decode lse"
    rows = _needle_rows(w)
    Or, lr = oracle_decode_parallel(w, rows)
    check_rows(O, lse, Or, lr, rows=rows, what="long_context_gqa L=1,048,576")
    check_rows(None, lse_e, None, lr, rows=rows, what="energy only, L=1,048,576")
    for (_, kvh, n) in w.notes["needles"]:
        assert 29.0 < lse[0, 0, w.G * kvh] < 31.0
    zrows = rows[:4]
    Fr = oracle.energy_rows(w.q, w.k, w.v, w.kv_lens, w.scale, inputs.bf16_to_f32(zeta),
                            rows=zrows)
    check_rows(None, F, None, Fr, rows=zrows, what="F(zeta), L=1,048,576")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_long_context_5m_needle():
    w = inputs.long_context_gqa(L=5_120_000, seed=3)
    say("generated 5.12M-token cache")
    q, k, v, lens = workload_tensors(w)
    O, lse = binding.decode(q, k, v, lens)
    torch.cuda.synchronize()
    O, lse = O.cpu().numpy(), lse.cpu().numpy()
    del q, k, v
    torch.cuda.empty_cache()
    # every needle row (all eight KV-head groups) and two other heads
    rows = _needle_rows(w, extra_heads=(1, 29))
    Or, lr = oracle_decode_parallel(w, rows)
    check_rows(O, lse, Or, lr, rows=rows, what="long_context_gqa L=5,120,000")
    # the needle dominates: O is its V row up to the weight left to the others
    for (_, kvh, n) in w.notes["needles"]:
        h = w.G * kvh
        assert 29.0 < lse[0, 0, h] < 31.0
        vn = w.values("v")[0, kvh, n]
        assert np.abs(O[0, 0, h] - vn).max() < 0.05
    lit = inputs.long_context_gqa(L=200_000, seed=3, literal_c=6.0)
    O2, l2 = run_decode(lit)
    rows2 = _needle_rows(lit)
    Or2, lr2 = oracle_decode(lit, rows=rows2)
    check_rows(O2, l2, Or2, lr2, rows=rows2, what="needle with the literal constant 6")


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_llama31_70b_ragged_full_size():
    w = inputs.llama31_70b_ragged(seed=5)
    say(f"lengths {w.kv_lens.tolist()}")
    O, lse = run_decode(w)
    # every sequence, one KV-head group of each (all 32 of its rows), and a
    # second group for the longest and the shortest sequence
    rng = np.random.default_rng(0)
    picks = [(b, int(rng.integers(0, w.Hkv))) for b in range(w.B)]
    for b in (int(np.argmax(w.kv_lens)), int(np.argmin(w.kv_lens))):
        picks.append((b, (dict(picks)[b] + 1) % w.Hkv))
    rows = []
    for b, kvh in picks:
        rows += [(b, i, h) for i in range(w.q_len) for h in range(kvh * w.G, (kvh + 1) * w.G)]
    Or, lr = oracle_decode_parallel(w, rows)
    check_rows(O, lse, Or, lr, rows=rows, what="llama31_70b_ragged (sampled groups)")


def test_llama31_70b_ragged_small():
    w = inputs.llama31_70b_ragged(seed=5, L_max=6000, L_lo=100, B=5)
    O, lse = run_decode(w)
    Or, lr = oracle_decode(w)
    check_rows(O, lse, Or, lr, what="ragged 70B-shaped, small lengths")


# ----------------------------------------------------------------------------
# Bifurcated shared-prefix batch
# ----------------------------------------------------------------------------
def run_bifurcated(w):
    O, lse = binding.decode_bifurcated(dev(w.q), dev(w.kp), dev(w.vp), dev(w.ks), dev(w.vs),
                                       scale=w.scale)
    torch.cuda.synchronize()
    return O.cpu().numpy(), lse.cpu().numpy()


def test_bifurcated_small():
    w = inputs.bifurcated_prefix(seed=41, S=5, Lp=1000, Ls=77)
    O, lse = run_bifurcated(w)
    Or, lr = oracle.attend_bifurcated(w.q, w.kp, w.vp, w.ks, w.vs, w.scale)
    check_rows(O[:, None], lse[:, None], Or[:, None], lr[:, None], what="bifurcated small")


def test_bifurcated_degenerate_parts():
    for Lp, Ls in ((0, 50), (300, 0), (0, 0), (1, 1)):
        w = inputs.bifurcated_prefix(seed=42, S=3, Hq=8, Hkv=2, D=64, Lp=Lp, Ls=Ls)
        O, lse = run_bifurcated(w)
        Or, lr = oracle.attend_bifurcated(w.q, w.kp, w.vp, w.ks, w.vs, w.scale)
        check_rows(O[:, None], lse[:, None], Or[:, None], lr[:, None], what=f"bifurcated Lp={Lp} Ls={Ls}")


BIF_MANY = [
    # S, Hq, Hkv, D, Lp, Ls: many samples (at least one sample x KV head per CU)
    (32, 32, 8, 128, 1000, 77),
    (64, 8, 4, 64, 0, 50),       # no prefix: the suffix alone
    (32, 16, 8, 128, 300, 1),    # one suffix token
    (32, 32, 8, 128, 700, 0),    # no suffix
    (32, 128, 8, 128, 500, 100),  # 16 rows per KV head: the suffix runs on the matrix cores
]


@pytest.mark.parametrize("case", BIF_MANY, ids=[f"S{c[0]}_Hq{c[1]}_Hkv{c[2]}_D{c[3]}_Lp{c[4]}_Ls{c[5]}" for c in BIF_MANY])
def test_bifurcated_many_samples(case):
    S, Hq, Hkv, D, Lp, Ls = case
    say(f"bifurcated {case}")
    w = inputs.bifurcated_prefix(seed=43 + Ls, S=S, Hq=Hq, Hkv=Hkv, D=D, Lp=Lp, Ls=Ls)
    O, lse = run_bifurcated(w)
    Or, lr = oracle.attend_bifurcated(w.q, w.kp, w.vp, w.ks, w.vs, w.scale)
    check_rows(O[:, None], lse[:, None], Or[:, None], lr[:, None], what=f"bifurcated {case}")


def test_prepared_bifurcated_call_matches_the_plain_call():
    """BifurcatedCall (set up once, run repeatedly) gives decode_bifurcated's
    result bit for bit, on every run."""
    w = inputs.bifurcated_prefix(seed=44, S=32, Lp=2000, Ls=300)
    t = [dev(x) for x in (w.q, w.kp, w.vp, w.ks, w.vs)]
    O0, lse0 = binding.decode_bifurcated(*t, scale=w.scale)
    call = binding.BifurcatedCall(*t, scale=w.scale)
    for _ in range(2):
        O1, lse1 = call.run()
        torch.cuda.synchronize()
        assert torch.equal(O0, O1) and torch.equal(lse0, lse1)


def test_graph_replays_match_eager_calls():
    """A decode (split + merge) and two bifurcated calls captured into one
    HIP graph (prepared calls bound to the capturing stream; the library
    launches kernels only, no memset, no allocation) and replayed three
    times, with eager work and synchronisation between the replays: every
    replay gives the eager results bit for bit.  The second bifurcated call
    has 64 samples, so it runs the one-launch shared-prefix kernel."""
    w = inputs.make_decode("graph", 77, B=2, q_len=1, Hq=32, Hkv=8, D=128, L_max=3000,
                           kv_lens=[3000, 1500], nan_pad=True)
    q, k, v, lens = workload_tensors(w)
    O0, lse0 = binding.decode(q, k, v, lens, scale=w.scale)
    calls = []
    for wb in (inputs.bifurcated_prefix(seed=45, S=8, Lp=700, Ls=90),
               inputs.bifurcated_prefix(seed=46, S=64, Lp=1024, Ls=64)):
        tb = [dev(x) for x in (wb.q, wb.kp, wb.vp, wb.ks, wb.vs)]
        calls.append((tb, wb.scale) + binding.decode_bifurcated(*tb, scale=wb.scale))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        ph = binding.Phases(q, k, v, lens, scale=w.scale)
        bcs = [binding.BifurcatedCall(*tb, scale=sc) for tb, sc, _, _ in calls]
        ph.partials()
        ph.merge()
        for bc in bcs:
            bc.run()
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        ph.partials()
        ph.merge()
        for bc in bcs:
            bc.run()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in [ph.out, ph.lse] + [x for bc in bcs for x in (bc.out, bc.lse)]:
            t.fill_(float("nan"))
        binding.decode(q, k, v, lens, scale=w.scale)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ph.out, O0) and torch.equal(ph.lse, lse0), f"decode, replay {rep}"
        for i, (bc, (_, _, Ob0, lseb0)) in enumerate(zip(bcs, calls)):
            assert torch.equal(bc.out, Ob0) and torch.equal(bc.lse, lseb0), \
                f"bifurcated call {i}, replay {rep}"


# The one-launch shared-prefix kernel in each of its forms (64 samples x 4
# query heads per KV head: the prefix takes 256-row blocks): CUs split with
# most on the prefix, CUs split with most on the suffix, and every workgroup
# on both parts (a suffix too short to be worth a round of the XCDs).
BIF_FORMS = [("split_prefix_heavy", 4096, 8), ("split_suffix_heavy", 1024, 1024),
             ("shared", 4096, 2)]


@pytest.mark.parametrize("form,Lp,Ls", BIF_FORMS, ids=[f[0] for f in BIF_FORMS])
def test_bifurcated_forms(form, Lp, Ls):
    say(f"bifurcated form {form} Lp={Lp} Ls={Ls}")
    w = inputs.bifurcated_prefix(seed=47 + Ls, Lp=Lp, Ls=Ls)
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    lib = binding.load_testing_library()
    d = binding.AttnBifDesc(num_samples=w.S, num_q_heads=w.Hq, num_kv_heads=w.Hkv,
                            head_dim=w.D, prefix_len=Lp, suffix_len=Ls, scale=w.scale, dtype=0)
    f, p, s = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
    assert lib.attn_testing_bifurcated_form(ctypes.byref(d), cu, ctypes.byref(f), ctypes.byref(p),
                                            ctypes.byref(s)) == 0
    assert f.value == 1
    if form == "shared":
        assert p.value == s.value == cu
    else:
        assert p.value + s.value == cu and (p.value > s.value) == (form == "split_prefix_heavy")
    O, lse = run_bifurcated(w)
    Or, lr = oracle.attend_bifurcated(w.q, w.kp, w.vp, w.ks, w.vs, w.scale)
    check_rows(O[:, None], lse[:, None], Or[:, None], lr[:, None], what=f"bifurcated {form}")


def test_bifurcated_full_size():
    w = inputs.bifurcated_prefix(seed=4)
    O, lse = run_bifurcated(w)
    Or, lr = oracle.attend_bifurcated(w.q, w.kp, w.vp, w.ks, w.vs, w.scale)
    check_rows(O[:, None], lse[:, None], Or[:, None], lr[:, None], what="bifurcated_prefix full")


# Non-positive scales: the MFMA kernels move a negative scale into Q (negating
# bf16 is exact) and treat a zero scale as zero logits; the vector-ALU kernel
# applies the scale as given.  All three kernels, against the oracle.
@pytest.mark.parametrize("scale", [-0.07, 0.0])
@pytest.mark.parametrize("shape", [(2, 1, 8, 2, 700), (2, 4, 32, 4, 900), (1, 8, 64, 2, 1200)],
                         ids=["valu", "mfma32", "rows"])
def test_non_positive_scale(scale, shape):
    B, q_len, Hq, Hkv, L = shape
    w = inputs.make_decode("negscale", 900 + L, B=B, q_len=q_len, Hq=Hq, Hkv=Hkv, D=128, L_max=L,
                           kv_lens=[L, L // 2 + 3][:B], causal=q_len > 1, scale=scale,
                           nan_pad=True)
    O, lse = run_decode(w)
    Or, lr = oracle_decode(w)
    check_rows(O, lse, Or, lr, what=f"scale {scale} {shape}")
