"""CPU fp64 oracle for exact split-KV attention decoding.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library.
"""
from .attention import (attend, attend_anchor_blocks, attend_bifurcated, attend_row,
                        chunk_partial, energy, energy_rows, finalize, merge, visible)
from .paging import attend_paged, gather

__all__ = ["attend", "attend_anchor_blocks", "attend_bifurcated", "attend_paged", "attend_row", "chunk_partial",
           "energy", "energy_rows", "finalize", "gather", "merge", "visible"]
