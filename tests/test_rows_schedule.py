"""The shared-tile MFMA kernel's LDS schedule has no cross-wave hazard.

The kernel keeps kRowsBufs K/V tile buffers (tile x in buffer x % kRowsBufs),
stores tile t + kStoreAhead in iteration t, reads V of tile t and K of tile
t + 2 in iteration t, and places a workgroup barrier only after odd
iterations (plus one after the prologue and one after the loop).  Waves run
unordered between barriers, so every access is placed in an epoch (the number
of barriers before it) and the schedule is safe when

  * each read of a tile lies in a later epoch than the store of that tile
    into its buffer (read after write), and
  * the next store into that buffer lies in a later epoch than every read
    of the tile it replaces (write after read).

The two constants are read from the kernel source, so a change there is
checked here.  CPU only.
"""
import os
import re

import pytest

SRC = os.path.join(os.path.dirname(__file__), "..", "long_context_exact_split_amd", "csrc",
                   "mfma_piece.h")


def _constants():
    text = open(SRC).read()
    bufs = int(re.search(r"constexpr int kRowsBufs = (\d+);", text).group(1))
    ahead = int(re.search(r"constexpr int kStoreAhead = (\d+);", text).group(1))
    unroll = int(re.search(r"constexpr int U = (\d+);", text).group(1))
    odd_only = "if (k & 1) __syncthreads();" in text
    return bufs, ahead, unroll, odd_only


def _events(n_tiles, bufs, ahead, odd_only):
    """(epoch, kind, tile, buffer) of one workgroup's pass over n_tiles tiles."""
    ev = []
    epoch = 0
    for x in range(ahead):  # prologue stores, then a barrier
        ev.append((epoch, "w", x, x % bufs))
    epoch += 1
    ev.append((epoch, "r", 0, 0))           # S^T of tile 0
    ev.append((epoch, "r", 1, 1 % bufs))    # S^T of tile 1
    for t in range(n_tiles - 1):
        ev.append((epoch, "r", t, t % bufs))              # V of tile t
        ev.append((epoch, "r", t + 2, (t + 2) % bufs))    # K of tile t + 2
        ev.append((epoch, "w", t + ahead, (t + ahead) % bufs))
        if not odd_only or t % 2 == 1:
            epoch += 1
    ev.append((epoch, "r", n_tiles - 1, (n_tiles - 1) % bufs))  # the last tile's V
    return ev


def _check(ev):
    writes = {}  # buffer -> list of (epoch, tile) in program order
    for e, kind, tile, b in ev:
        if kind == "w":
            writes.setdefault(b, []).append((e, tile))
    for e, kind, tile, b in ev:
        if kind != "r":
            continue
        ws = writes[b]
        idx = [i for i, (_, x) in enumerate(ws) if x == tile]
        assert idx, f"tile {tile} read from buffer {b} but never stored there"
        i = idx[-1]
        assert ws[i][0] < e, f"tile {tile}: stored in epoch {ws[i][0]}, read in epoch {e}"
        if i + 1 < len(ws):
            assert ws[i + 1][0] > e, (f"buffer {b}: tile {ws[i + 1][1]} stored in epoch "
                                      f"{ws[i + 1][0]}, tile {tile} still read in epoch {e}")


def test_constants_found():
    bufs, ahead, unroll, odd_only = _constants()
    assert bufs >= 3 and ahead >= 3 and unroll % 2 == 0 and odd_only


@pytest.mark.parametrize("n_tiles", list(range(1, 41)))
def test_schedule_has_no_hazard(n_tiles):
    bufs, ahead, _, odd_only = _constants()
    _check(_events(n_tiles, bufs, ahead, odd_only))


def test_checker_catches_unsafe_schedules():
    """The model rejects schedules one step too tight, so it is not vacuous."""
    bufs, ahead, _, _ = _constants()
    with pytest.raises(AssertionError):  # too few buffers: overwrite before the last read
        _check(_events(20, ahead + 1, ahead, True))
    with pytest.raises(AssertionError):  # stored too late: K read in the same epoch
        _check(_events(20, bufs, 3, True))
    _check(_events(20, 4, 3, False))     # the per-iteration barrier form is safe too
