"""Host check of the lane choreography of the vector-ALU kernel's energy path.

The kernel reduce-scatters the per-row partial dot products of a key row's
LPK lanes with DPP steps (quad xor 1, quad xor 2, half-row mirror, row
mirror, xor 16).  Emulating those lane permutations here in float32, with the
same operand order as the kernel, checks that every lane ends with exactly
(bit for bit) the all-reduce sum of the row scatter_row assigns it, and that
lanes 0 .. RB-1 of a key row own distinct rows (they write the records)."""
import numpy as np
import pytest

QUAD_XOR1 = [i ^ 1 for i in range(64)]
QUAD_XOR2 = [i ^ 2 for i in range(64)]
HALF_MIRROR = [(i & ~7) | (7 - (i & 7)) for i in range(64)]
ROW_MIRROR = [(i & ~15) | (15 - (i & 15)) for i in range(64)]
XOR16 = [i ^ 16 for i in range(64)]


def pull(v, perm):
    return np.array([v[perm[i]] for i in range(64)], dtype=np.float32)


def group_sum(x, lpk):
    steps = [QUAD_XOR1, QUAD_XOR2, HALF_MIRROR, ROW_MIRROR, XOR16]
    n = {8: 3, 16: 4, 32: 5}[lpk]
    for p in steps[:n]:
        x = (x + pull(x, p)).astype(np.float32)
    return x


def quad_pos(kl):
    return (kl & 3) ^ (3 if (kl >> 2) & 1 else 0)


def scatter_row(kl, lpk, rb):
    pq = quad_pos(kl)
    r = 0
    if rb >= 2:
        r += (pq & 1) * (rb // 2)
    if rb >= 4:
        r += ((pq >> 1) & 1) * (rb // 4)
    if rb >= 8:
        r += (((kl >> 2) ^ (kl >> 3)) & 1) if lpk >= 16 else ((kl >> 2) & 1)
    return r


def row_scatter_sum(x, lpk, rb):
    """x: [64 lanes][rb] float32 -> [64] (one row per lane), kernel step order."""
    kl = np.arange(64) % lpk
    v = [x[:, r].copy() for r in range(rb)]

    def step(perm, up, half):
        nonlocal v
        out = []
        for k in range(half):
            keep = np.where(up, v[half + k], v[k]).astype(np.float32)
            send = np.where(up, v[k], v[half + k]).astype(np.float32)
            out.append((keep + pull(send, perm)).astype(np.float32))
        v = out

    pq = np.array([quad_pos(int(k)) for k in kl])
    if rb >= 2:
        step(QUAD_XOR1, (pq & 1).astype(bool), rb // 2)
    else:
        v[0] = (v[0] + pull(v[0], QUAD_XOR1)).astype(np.float32)
    if rb >= 4:
        step(QUAD_XOR2, ((pq >> 1) & 1).astype(bool), rb // 4)
    else:
        v[0] = (v[0] + pull(v[0], QUAD_XOR2)).astype(np.float32)
    if rb >= 8:
        up = (((kl >> 2) ^ (kl >> 3)) & 1) if lpk >= 16 else ((kl >> 2) & 1)
        step(HALF_MIRROR, up.astype(bool), 1)
    else:
        v[0] = (v[0] + pull(v[0], HALF_MIRROR)).astype(np.float32)
    if lpk >= 16:
        v[0] = (v[0] + pull(v[0], ROW_MIRROR)).astype(np.float32)
    if lpk >= 32:
        v[0] = (v[0] + pull(v[0], XOR16)).astype(np.float32)
    return v[0]


@pytest.mark.parametrize("lpk", [8, 16, 32])
@pytest.mark.parametrize("rb", [1, 2, 4, 8])
def test_reduce_scatter_matches_all_reduce_bitwise(lpk, rb):
    rng = np.random.default_rng(lpk * 10 + rb)
    for _ in range(20):
        x = (rng.standard_normal((64, rb)) * 10).astype(np.float32)
        full = np.stack([group_sum(x[:, r].copy(), lpk) for r in range(rb)], axis=1)
        got = row_scatter_sum(x, lpk, rb)
        for lane in range(64):
            r = scatter_row(lane % lpk, lpk, rb)
            assert got[lane].tobytes() == full[lane, r].tobytes(), (lane, r)
    owners = [scatter_row(k, lpk, rb) for k in range(rb)]
    assert sorted(owners) == list(range(rb))
