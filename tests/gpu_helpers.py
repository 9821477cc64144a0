"""Helpers for the GPU parity tests: device upload and the parity bar.

The bar: max |dO| <= 2e-3 and |dlse| <= 1e-4 * max(1, |lse|) against the fp64
oracle on the same bf16-rounded inputs; a row that sees no key must give
lse = -inf and O = 0 exactly; NaN is never acceptable.
"""
import sys

import numpy as np
import torch

O_TOL = 2e-3
LSE_RTOL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def workload_tensors(w):
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    lens = None
    if not (w.kv_lens == w.L_max).all():
        lens = torch.from_numpy(w.kv_lens.astype(np.int32)).cuda()
    return q, k, v, lens


def check_rows(O, lse, O_ref, lse_ref, rows=None, what=""):
    """Compare GPU outputs to the oracle on all rows (or the listed (b,i,h) rows)."""
    O = None if O is None else np.asarray(O, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    if rows is None:
        sel = np.ones(lse.shape, dtype=bool)
    else:
        sel = np.zeros(lse.shape, dtype=bool)
        for r in rows:
            sel[r] = True
    assert not np.isnan(lse[sel]).any(), f"{what}: NaN lse"
    if O is not None:
        assert not np.isnan(O[sel]).any(), f"{what}: NaN O"
    ref_inf = np.isneginf(lse_ref) & sel
    assert (lse[ref_inf] == -np.inf).all(), f"{what}: empty rows must give lse=-inf"
    fin = sel & ~ref_inf
    dl = np.abs(lse[fin] - lse_ref[fin])
    bound = LSE_RTOL * np.maximum(1.0, np.abs(lse_ref[fin]))
    worst_l = float((dl / bound).max()) if dl.size else 0.0
    assert (dl <= bound).all(), f"{what}: lse off by {dl.max():.3e} (ratio to bound {worst_l:.2f})"
    worst_o = 0.0
    if O is not None and O_ref is not None:
        if ref_inf.any():
            assert (O[ref_inf] == 0).all(), f"{what}: empty rows must give O=0"
        dO = np.abs(O[fin] - O_ref[fin])
        worst_o = float(dO.max()) if dO.size else 0.0
        assert worst_o <= O_TOL, f"{what}: max|dO| = {worst_o:.3e}"
    say(f"  {what}: rows={int(sel.sum())} max|dO|={worst_o:.2e} lse/bound={worst_l:.3f}")
    return worst_o, worst_l
