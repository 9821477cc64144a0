"""ctypes binding of ``libattn_decode.so`` (argument marshalling only).

Every step of the computation runs in the library's HIP kernels.  This module
checks tensor shapes/dtypes, allocates outputs and the workspace with torch
(device memory is the only thing torch provides), passes raw pointers and the
current HIP stream, and turns status codes into ``AttnError``.  If the library
is not built the functions raise; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libattn_decode.so"
# Test build: the same library plus the hooks of include/attn_decode_testing.h.
# ATTN_TESTING_LIB names another build of those hooks (the host sanitizer test).
TESTING_LIB_NAME = "libattn_decode_testing.so"

ATTN_BF16, ATTN_F32 = 0, 1
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_DTYPE",
          4: "ATTN_ERR_ALIGN", 5: "ATTN_ERR_WORKSPACE", 6: "ATTN_ERR_HIP",
          7: "ATTN_ERR_UNSUPPORTED", 8: "ATTN_ERR_VALUE", 9: "ATTN_ERR_SCRATCH"}
EXPORTS = ("attn_decode_plan", "attn_workspace_bytes", "attn_decode_energy", "attn_decode",
           "attn_decode_partials", "attn_decode_merge", "attn_decode_energy_zeta",
           "attn_decode_paged", "attn_decode_energy_paged", "attn_decode_partials_paged",
           "attn_bifurcated_workspace_bytes", "attn_decode_bifurcated",
           "attn_anchor_workspace_bytes", "attn_prefill_anchor", "attn_decode_static",
           "attn_merge_results", "attn_status_string")


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = STATUS.get(status, str(status))
        if _lib is not None:
            msg += ": " + _lib.attn_status_string(status).decode()
        super().__init__(f"{where}: {msg}")


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_len", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("max_kv_len", ctypes.c_int64), ("kv_lens", ctypes.c_void_p),
                ("scale", ctypes.c_float), ("chunk_len", ctypes.c_int32),
                ("dtype", ctypes.c_int)]


class AttnPlan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("rows_per_block", ctypes.c_int32), ("row_blocks", ctypes.c_int32),
                ("balanced", ctypes.c_int32), ("chunk_len", ctypes.c_int32),
                ("chunks_per_seq", ctypes.c_int32), ("threads_per_item", ctypes.c_int32),
                ("work_items", ctypes.c_int64), ("record_slots", ctypes.c_int64),
                ("cu_count", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class AttnBifDesc(ctypes.Structure):
    _fields_ = [("num_samples", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("prefix_len", ctypes.c_int64), ("suffix_len", ctypes.c_int64),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int)]


class AttnAnchorDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_len", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("anchor_len", ctypes.c_int64),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int)]


class AttnPagedKv(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("pages_per_seq", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int64),
                ("page_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("token_stride", ctypes.c_int64)]


_lib = None
_testing_lib = None
_lock = threading.Lock()


def library_path() -> str:
    """The product library next to this file; ATTN_LIB names another build of
    it (the bench's per-workgroup timing build), which must export the same
    entry points."""
    return os.environ.get("ATTN_LIB") or os.path.join(PKG, LIB_NAME)


def load_library():
    """Load the HIP library (raises AttnError-free RuntimeError if it is not built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run __graft_entry__.build() "
                               "(or python -m long_context_exact_split_amd.build)")
        lib = ctypes.CDLL(path)
        P, c = ctypes.POINTER, ctypes
        lib.attn_decode_plan.argtypes = [P(AttnDesc), c.c_int32, P(AttnPlan)]
        lib.attn_workspace_bytes.argtypes = [P(AttnDesc), P(c.c_size_t)]
        lib.attn_decode_energy.argtypes = [P(AttnDesc), c.c_void_p, c.c_void_p, c.c_void_p,
                                           c.c_void_p, c.c_size_t, c.c_void_p]
        lib.attn_decode.argtypes = [P(AttnDesc), c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                                    c.c_void_p, c.c_void_p, c.c_size_t, c.c_void_p]
        lib.attn_decode_partials.argtypes = [P(AttnDesc), c.c_void_p, c.c_void_p, c.c_void_p,
                                             c.c_void_p, c.c_size_t, c.c_void_p]
        lib.attn_decode_merge.argtypes = [P(AttnDesc), c.c_void_p, c.c_void_p, c.c_void_p,
                                          c.c_size_t, c.c_void_p]
        lib.attn_decode_energy_zeta.argtypes = [P(AttnDesc)] + [c.c_void_p] * 6 + [
            c.c_size_t, c.c_void_p]
        lib.attn_decode_paged.argtypes = [P(AttnDesc), P(AttnPagedKv)] + [c.c_void_p] * 6 + [
            c.c_size_t, c.c_void_p]
        lib.attn_decode_energy_paged.argtypes = [P(AttnDesc), P(AttnPagedKv)] + [
            c.c_void_p] * 4 + [c.c_size_t, c.c_void_p]
        lib.attn_decode_partials_paged.argtypes = [P(AttnDesc), P(AttnPagedKv)] + [
            c.c_void_p] * 4 + [c.c_size_t, c.c_void_p]
        lib.attn_bifurcated_workspace_bytes.argtypes = [P(AttnBifDesc), P(c.c_size_t)]
        lib.attn_anchor_workspace_bytes.argtypes = [P(AttnAnchorDesc), P(c.c_size_t)]
        lib.attn_prefill_anchor.argtypes = [P(AttnAnchorDesc)] + [c.c_void_p] * 8 + [
            c.c_size_t, c.c_void_p]
        lib.attn_decode_bifurcated.argtypes = [P(AttnBifDesc)] + [c.c_void_p] * 8 + [
            c.c_size_t, c.c_void_p]
        lib.attn_decode_static.argtypes = [P(AttnDesc)] + [c.c_void_p] * 6
        lib.attn_merge_results.argtypes = [c.c_int32, c.c_int64, c.c_int32] + [c.c_void_p] * 5
        for name in EXPORTS[:-1]:
            getattr(lib, name).restype = c.c_int
        lib.attn_status_string.argtypes = [c.c_int]
        lib.attn_status_string.restype = c.c_char_p
        _lib = lib
        return lib


def load_testing_library():
    """Load the test build (partition and check hooks; never used by the product path)."""
    global _testing_lib
    with _lock:
        if _testing_lib is not None:
            return _testing_lib
        path = os.environ.get("ATTN_TESTING_LIB") or os.path.join(PKG, TESTING_LIB_NAME)
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        P, c = ctypes.POINTER, ctypes
        lib.attn_testing_pieces.argtypes = [P(AttnDesc), c.c_void_p, c.c_int32, c.c_int64,
                                            c.c_void_p, c.c_int64]
        lib.attn_testing_pieces.restype = c.c_int64
        lib.attn_testing_segment_slots.argtypes = [P(AttnDesc), c.c_void_p, c.c_int32, c.c_int64,
                                                   c.c_void_p]
        lib.attn_testing_segment_slots.restype = c.c_int
        lib.attn_testing_anchor_fuses.argtypes = [P(AttnAnchorDesc), c.c_int32]
        lib.attn_testing_anchor_fuses.restype = c.c_int32
        lib.attn_testing_plan.argtypes = [P(AttnDesc), c.c_int32, P(AttnPlan)]
        lib.attn_testing_plan.restype = c.c_int
        lib.attn_testing_check_decode.argtypes = [P(AttnDesc), P(AttnPagedKv)] + [
            c.c_void_p] * 5 + [c.c_int32, c.c_int32]
        lib.attn_testing_check_decode.restype = c.c_int
        lib.attn_testing_check_bifurcated.argtypes = [P(AttnBifDesc), c.c_int32, P(c.c_size_t)]
        lib.attn_testing_check_bifurcated.restype = c.c_int
        lib.attn_testing_bifurcated_form.argtypes = [P(AttnBifDesc), c.c_int32, P(c.c_int32),
                                                     P(c.c_int64), P(c.c_int64)]
        lib.attn_testing_bifurcated_form.restype = c.c_int
        if hasattr(lib, "attn_testing_prefill_anchor_unfused"):  # absent in host-only builds
            lib.attn_testing_prefill_anchor_unfused.argtypes = [P(AttnAnchorDesc)] + [
                c.c_void_p] * 8 + [c.c_size_t, c.c_void_p]
            lib.attn_testing_prefill_anchor_unfused.restype = c.c_int
        _testing_lib = lib
        return lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise AttnError(status, where)


def make_desc(*, batch, q_len, num_q_heads, num_kv_heads, head_dim, max_kv_len, kv_lens_ptr=0,
              scale=None, causal=False, chunk_len=0, dtype=ATTN_BF16) -> AttnDesc:
    d = AttnDesc()
    d.batch, d.q_len, d.num_q_heads, d.num_kv_heads = batch, q_len, num_q_heads, num_kv_heads
    d.head_dim, d.causal, d.max_kv_len = head_dim, int(bool(causal)), max_kv_len
    d.kv_lens = kv_lens_ptr or None
    d.scale = (1.0 / math.sqrt(head_dim) if head_dim > 0 else 1.0) if scale is None else scale
    d.chunk_len, d.dtype = chunk_len, dtype
    return d


def plan(desc: AttnDesc, cu_count: int = 0) -> dict:
    """The partitioner's decision (pure host code when cu_count > 0)."""
    lib = load_library()
    p = AttnPlan()
    _check(lib.attn_decode_plan(ctypes.byref(desc), cu_count, ctypes.byref(p)), "attn_decode_plan")
    return p.as_dict()


def testing_plan(desc: AttnDesc, cu_count: int) -> dict:
    """The plan through the test build's host-only hook (same arithmetic as plan())."""
    p = AttnPlan()
    _check(load_testing_library().attn_testing_plan(ctypes.byref(desc), cu_count, ctypes.byref(p)),
           "attn_testing_plan")
    return p.as_dict()


def testing_pieces(desc: AttnDesc, lens, cu_count: int, w: int):
    """Host view of workgroup w's pieces: [(segment, t0, t1, slot), ...]."""
    import numpy as np
    lib = load_testing_library()
    arr = None if lens is None else np.ascontiguousarray(lens, dtype=np.int32)
    cap = 64
    while True:
        out = np.zeros(4 * cap, dtype=np.int64)
        n = lib.attn_testing_pieces(ctypes.byref(desc), None if arr is None else arr.ctypes.data,
                                    cu_count, w, out.ctypes.data, cap)
        if n < 0:
            raise AttnError(int(-n), "attn_testing_pieces")
        if n <= cap:
            return [tuple(int(x) for x in out[4 * i:4 * i + 4]) for i in range(n)]
        cap = int(n)


def testing_anchor_fuses(desc: "AttnAnchorDesc", cu_count: int) -> bool:
    """Whether attn_prefill_anchor finalises rows in its local split for this shape."""
    r = load_testing_library().attn_testing_anchor_fuses(ctypes.byref(desc), cu_count)
    if r < 0:
        raise AttnError(int(-r), "attn_testing_anchor_fuses")
    return bool(r)


def testing_segment_slots(desc: AttnDesc, lens, cu_count: int, segment: int):
    import numpy as np
    lib = load_testing_library()
    arr = None if lens is None else np.ascontiguousarray(lens, dtype=np.int32)
    out = np.zeros(3, dtype=np.int64)
    _check(lib.attn_testing_segment_slots(ctypes.byref(desc), None if arr is None else arr.ctypes.data,
                                          cu_count, segment, out.ctypes.data),
           "attn_testing_segment_slots")
    return tuple(int(x) for x in out)


def workspace_bytes(desc: AttnDesc) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.attn_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)), "attn_workspace_bytes")
    return n.value


# ----------------------------------------------------------------------------
# torch-facing wrappers
# ----------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported element type {t.dtype} (bfloat16 or float32)")


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream_ptr(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device, workspace):
    torch = _torch()
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.device != device or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on {device}")
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _output(t, shape, device, name):
    """A caller-supplied output (float32, contiguous, on `device`, of `shape`)
    or a new one.  Checked here because the library sees only a pointer."""
    torch = _torch()
    if t is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    if t.dtype != torch.float32 or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor on {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    return t


def _decode_desc(q, k, kv_lens, scale, causal, chunk_len) -> AttnDesc:
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, q_len, Hq, D] and k/v [B, Hkv, L, D]")
    B, q_len, Hq, D = q.shape
    Bk, Hkv, L, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)}")
    if kv_lens is not None:
        torch = _torch()
        if kv_lens.dtype != torch.int32 or kv_lens.numel() != B or kv_lens.device != q.device:
            raise ValueError("kv_lens must be int32[B] on the device of q")
        if not kv_lens.is_contiguous():
            raise ValueError("kv_lens must be contiguous")
    return make_desc(batch=B, q_len=q_len, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                     max_kv_len=L, kv_lens_ptr=_ptr(kv_lens), scale=scale, causal=causal,
                     chunk_len=chunk_len, dtype=_dtype_code(q))


def _check_tensors(*ts):
    ref = ts[0]
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("q, k and v must share dtype and device")


def decode(q, k, v, kv_lens=None, *, scale: Optional[float] = None, causal: bool = False,
           chunk_len: int = 0, out=None, lse=None, workspace=None) -> Tuple[object, object]:
    """Exact attention decode: returns (O float32 [B,q_len,Hq,D], lse float32 [B,q_len,Hq])."""
    torch = _torch()
    lib = load_library()
    _check_tensors(q, k, v)
    if v.shape != k.shape:
        raise ValueError("v must have the shape of k")
    desc = _decode_desc(q, k, kv_lens, scale, causal, chunk_len)
    B, q_len, Hq, D = q.shape
    with torch.cuda.device(q.device):
        out = _output(out, (B, q_len, Hq, D), q.device, "out")
        lse = _output(lse, (B, q_len, Hq), q.device, "lse")
        ws = _workspace(workspace_bytes(desc), q.device, workspace)
        nbytes = 0 if ws is None else ws.numel() * ws.element_size()
        _check(lib.attn_decode(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                               _ptr(lse), _ptr(ws), nbytes, _stream_ptr(q.device)), "attn_decode")
    return out, lse


def decode_static(q, k, v, kv_lens=None, *, scale: Optional[float] = None, causal: bool = False,
                  chunk_len: int = 0, out=None, lse=None) -> Tuple[object, object]:
    """attn_decode_static: as decode(), with the partial records in the
    library's own device array (no workspace; the C call allocates nothing).
    Calls that overlap on one GPU race on that array."""
    torch = _torch()
    lib = load_library()
    _check_tensors(q, k, v)
    if v.shape != k.shape:
        raise ValueError("v must have the shape of k")
    desc = _decode_desc(q, k, kv_lens, scale, causal, chunk_len)
    B, q_len, Hq, D = q.shape
    with torch.cuda.device(q.device):
        out = _output(out, (B, q_len, Hq, D), q.device, "out")
        lse = _output(lse, (B, q_len, Hq), q.device, "lse")
        _check(lib.attn_decode_static(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                      _ptr(lse), _stream_ptr(q.device)), "attn_decode_static")
    return out, lse


class Phases:
    """The two phases of one decode call on fixed buffers: ``partials()``
    launches the split-KV kernel (records into the workspace), ``merge()``
    the merge + normalisation.  Used to time the kernels separately.  With
    ``v`` None the call is energy only (lse, no O).  With ``paged`` (a
    ``PagedCache``) k and v are its pools."""

    def __init__(self, q, k, v, kv_lens=None, *, scale=None, causal=False, chunk_len=0,
                 paged=None):
        torch = _torch()
        self.lib = load_library()
        _check_tensors(q, k, v)
        self.paged = paged
        if paged is None:
            self.desc = _decode_desc(q, k, kv_lens, scale, causal, chunk_len)
        else:
            self.desc = _paged_desc(q, paged, kv_lens, scale, causal, chunk_len)
        B, q_len, Hq, D = q.shape
        self.q, self.k, self.v, self.kv_lens = q, k, v, kv_lens
        self.out = (None if v is None else
                    torch.empty((B, q_len, Hq, D), dtype=torch.float32, device=q.device))
        self.lse = torch.empty((B, q_len, Hq), dtype=torch.float32, device=q.device)
        self.ws = _workspace(workspace_bytes(self.desc), q.device, None)
        self.nbytes = 0 if self.ws is None else self.ws.numel()
        self.plan = plan(self.desc)
        self.stream = _stream_ptr(q.device)

    def partials(self):
        if self.paged is not None:
            _check(self.lib.attn_decode_partials_paged(
                ctypes.byref(self.desc), ctypes.byref(self.paged.kv), _ptr(self.q), _ptr(self.k),
                _ptr(self.v), _ptr(self.ws), self.nbytes, self.stream),
                "attn_decode_partials_paged")
            return
        _check(self.lib.attn_decode_partials(ctypes.byref(self.desc), _ptr(self.q), _ptr(self.k),
                                             _ptr(self.v), _ptr(self.ws), self.nbytes,
                                             self.stream), "attn_decode_partials")

    def merge(self):
        _check(self.lib.attn_decode_merge(ctypes.byref(self.desc), _ptr(self.out), _ptr(self.lse),
                                          _ptr(self.ws), self.nbytes, self.stream),
               "attn_decode_merge")


def merge_results(o_parts, lse_parts, *, out=None, lse=None):
    """Merge results computed over disjoint shares of the keys (one share per
    device in a sequence-sharded decode): o_parts float32 [n, ..., D] and
    lse_parts float32 [n, ...] (the n results of the same rows) give O
    [..., D] and lse [...] over all the keys (attn_merge_results)."""
    torch = _torch()
    lib = load_library()
    if o_parts.dim() < 2 or lse_parts.shape != o_parts.shape[:-1]:
        raise ValueError("o_parts must be [n, ..., D] and lse_parts [n, ...] with the same rows")
    for t, name in ((o_parts, "o_parts"), (lse_parts, "lse_parts")):
        if (not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous()
                or t.device != o_parts.device):
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor on {o_parts.device}")
    n, D = o_parts.shape[0], o_parts.shape[-1]
    rows = lse_parts[0].numel() if n > 0 else 0
    with torch.cuda.device(o_parts.device):
        out = _output(out, tuple(o_parts.shape[1:]), o_parts.device, "out")
        lse = _output(lse, tuple(lse_parts.shape[1:]), o_parts.device, "lse")
        _check(lib.attn_merge_results(n, rows, D, _ptr(o_parts), _ptr(lse_parts), _ptr(out),
                                      _ptr(lse), _stream_ptr(o_parts.device)),
               "attn_merge_results")
    return out, lse


def merge_energies(lse_parts, *, lse=None):
    """The lse-only form of merge_results: lse_parts float32 [n, ...] (the
    energies of n disjoint shares of the keys) give lse [...] over all of
    them, ln sum_p e^(lse_p)."""
    torch = _torch()
    lib = load_library()
    if lse_parts.dim() < 1:
        raise ValueError("lse_parts must be [n, ...]")
    if not lse_parts.is_cuda or lse_parts.dtype != torch.float32 or not lse_parts.is_contiguous():
        raise ValueError("lse_parts must be a contiguous float32 GPU tensor")
    n = lse_parts.shape[0]
    rows = lse_parts[0].numel() if n > 0 else 0
    with torch.cuda.device(lse_parts.device):
        lse = _output(lse, tuple(lse_parts.shape[1:]), lse_parts.device, "lse")
        _check(lib.attn_merge_results(n, rows, 64, None, _ptr(lse_parts), None, _ptr(lse),
                                      _stream_ptr(lse_parts.device)), "attn_merge_results")
    return lse


def decode_energy(q, k, kv_lens=None, *, scale: Optional[float] = None, causal: bool = False,
                  chunk_len: int = 0, lse=None, workspace=None):
    """Energy only (reads K, not V): returns lse float32 [B, q_len, Hq]."""
    torch = _torch()
    lib = load_library()
    _check_tensors(q, k)
    desc = _decode_desc(q, k, kv_lens, scale, causal, chunk_len)
    B, q_len, Hq, D = q.shape
    with torch.cuda.device(q.device):
        lse = _output(lse, (B, q_len, Hq), q.device, "lse")
        ws = _workspace(workspace_bytes(desc), q.device, workspace)
        nbytes = 0 if ws is None else ws.numel() * ws.element_size()
        _check(lib.attn_decode_energy(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(lse), _ptr(ws),
                                      nbytes, _stream_ptr(q.device)), "attn_decode_energy")
    return lse


def decode_energy_zeta(q, k, v, zeta, kv_lens=None, *, scale: Optional[float] = None,
                       causal: bool = False, chunk_len: int = 0, lse=None, workspace=None):
    """F(zeta) = ln sum_t exp(scale q.k_t + zeta.v_t) per row: float32 [B, q_len, Hq].
    ``zeta`` has the shape and dtype of ``q``."""
    torch = _torch()
    lib = load_library()
    _check_tensors(q, k, v, zeta)
    if v.shape != k.shape or zeta.shape != q.shape:
        raise ValueError("v must have the shape of k and zeta the shape of q")
    desc = _decode_desc(q, k, kv_lens, scale, causal, chunk_len)
    B, q_len, Hq, D = q.shape
    with torch.cuda.device(q.device):
        lse = _output(lse, (B, q_len, Hq), q.device, "lse")
        ws = _workspace(workspace_bytes(desc), q.device, workspace)
        nbytes = 0 if ws is None else ws.numel() * ws.element_size()
        _check(lib.attn_decode_energy_zeta(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(zeta), _ptr(lse), _ptr(ws), nbytes,
                                           _stream_ptr(q.device)), "attn_decode_energy_zeta")
    return lse


# ----------------------------------------------------------------------------
# Paged KV caches
# ----------------------------------------------------------------------------
class PagedCache:
    """K/V pools of fixed-size pages plus a block table (device tensors).

    ``layout`` "head_major": pools [num_pages, Hkv, P, D]; "token_major":
    [num_pages, P, Hkv, D].  ``block_table``: int32 [B, pages_per_seq].
    ``max_kv_len`` defaults to pages_per_seq * P."""

    def __init__(self, k_pool, v_pool, block_table, *, layout="head_major", max_kv_len=None):
        torch = _torch()
        if layout not in ("head_major", "token_major"):
            raise ValueError("layout must be 'head_major' or 'token_major'")
        if k_pool.dim() != 4 or (v_pool is not None and v_pool.shape != k_pool.shape):
            raise ValueError("pools must be 4-d and of one shape")
        if block_table.dtype != torch.int32 or block_table.dim() != 2:
            raise ValueError("block_table must be int32 [B, pages_per_seq]")
        if not block_table.is_contiguous() or block_table.device != k_pool.device:
            raise ValueError("block_table must be contiguous and on the pools' device")
        n, a, b, D = k_pool.shape
        Hkv, P = (a, b) if layout == "head_major" else (b, a)
        self.k_pool, self.v_pool, self.block_table = k_pool, v_pool, block_table
        self.layout, self.num_kv_heads, self.page_size, self.head_dim = layout, Hkv, P, D
        self.pages_per_seq = block_table.shape[1]
        self.max_kv_len = self.pages_per_seq * P if max_kv_len is None else int(max_kv_len)
        kv = AttnPagedKv()
        kv.block_table = _ptr(block_table) or None
        kv.pages_per_seq, kv.page_size, kv.num_pages = self.pages_per_seq, P, n
        kv.page_stride = Hkv * P * D
        kv.head_stride, kv.token_stride = (P * D, D) if layout == "head_major" else (D, Hkv * D)
        self.kv = kv


def _paged_desc(q, paged: PagedCache, kv_lens, scale, causal, chunk_len) -> AttnDesc:
    if q.dim() != 4 or q.shape[3] != paged.head_dim:
        raise ValueError("q must be [B, q_len, Hq, D] with the pools' D")
    B, q_len, Hq, D = q.shape
    if paged.block_table.shape[0] != B:
        raise ValueError("block_table must have one row per sequence")
    if kv_lens is not None:
        torch = _torch()
        if kv_lens.dtype != torch.int32 or kv_lens.numel() != B or kv_lens.device != q.device:
            raise ValueError("kv_lens must be int32[B] on the device of q")
    return make_desc(batch=B, q_len=q_len, num_q_heads=Hq, num_kv_heads=paged.num_kv_heads,
                     head_dim=D, max_kv_len=paged.max_kv_len, kv_lens_ptr=_ptr(kv_lens),
                     scale=scale, causal=causal, chunk_len=chunk_len, dtype=_dtype_code(q))


def decode_paged(q, paged: PagedCache, kv_lens=None, *, scale: Optional[float] = None,
                 causal: bool = False, chunk_len: int = 0, out=None, lse=None, workspace=None):
    """Exact attention decode over a paged cache: (O float32 [B,q_len,Hq,D], lse)."""
    torch = _torch()
    lib = load_library()
    _check_tensors(q, paged.k_pool, paged.v_pool)
    desc = _paged_desc(q, paged, kv_lens, scale, causal, chunk_len)
    B, q_len, Hq, D = q.shape
    with torch.cuda.device(q.device):
        out = _output(out, (B, q_len, Hq, D), q.device, "out")
        lse = _output(lse, (B, q_len, Hq), q.device, "lse")
        ws = _workspace(workspace_bytes(desc), q.device, workspace)
        nbytes = 0 if ws is None else ws.numel() * ws.element_size()
        _check(lib.attn_decode_paged(ctypes.byref(desc), ctypes.byref(paged.kv), _ptr(q),
                                     _ptr(paged.k_pool), _ptr(paged.v_pool), _ptr(out), _ptr(lse),
                                     _ptr(ws), nbytes, _stream_ptr(q.device)), "attn_decode_paged")
    return out, lse


def decode_energy_paged(q, paged: PagedCache, kv_lens=None, *, scale: Optional[float] = None,
                        causal: bool = False, chunk_len: int = 0, lse=None, workspace=None):
    """Energy only over a paged cache (reads the K pool): lse float32 [B, q_len, Hq]."""
    torch = _torch()
    lib = load_library()
    _check_tensors(q, paged.k_pool)
    desc = _paged_desc(q, paged, kv_lens, scale, causal, chunk_len)
    B, q_len, Hq, D = q.shape
    with torch.cuda.device(q.device):
        lse = _output(lse, (B, q_len, Hq), q.device, "lse")
        ws = _workspace(workspace_bytes(desc), q.device, workspace)
        nbytes = 0 if ws is None else ws.numel() * ws.element_size()
        _check(lib.attn_decode_energy_paged(ctypes.byref(desc), ctypes.byref(paged.kv), _ptr(q),
                                            _ptr(paged.k_pool), _ptr(lse), _ptr(ws), nbytes,
                                            _stream_ptr(q.device)), "attn_decode_energy_paged")
    return lse


def bifurcated_desc(q, kp, ks, scale=None) -> AttnBifDesc:
    S, Hq, D = q.shape
    Hkv, Lp, Dp = kp.shape
    if ks.dim() != 4 or ks.shape[0] != S or ks.shape[1] != Hkv or ks.shape[3] != D or Dp != D:
        raise ValueError("q [S,Hq,D], k_prefix [Hkv,Lp,D], k_suffix [S,Hkv,Ls,D]")
    d = AttnBifDesc()
    d.num_samples, d.num_q_heads, d.num_kv_heads, d.head_dim = S, Hq, Hkv, D
    d.prefix_len, d.suffix_len = Lp, ks.shape[2]
    d.scale = (1.0 / math.sqrt(D)) if scale is None else scale
    d.dtype = _dtype_code(q)
    return d


def decode_bifurcated(q, k_prefix, v_prefix, k_suffix, v_suffix, *, scale: Optional[float] = None,
                      out=None, lse=None, workspace=None):
    """Shared-prefix batch sampling: returns (O float32 [S,Hq,D], lse float32 [S,Hq])."""
    torch = _torch()
    lib = load_library()
    _check_tensors(q, k_prefix, v_prefix, k_suffix, v_suffix)
    if v_prefix.shape != k_prefix.shape or v_suffix.shape != k_suffix.shape:
        raise ValueError("v tensors must match k tensors")
    desc = bifurcated_desc(q, k_prefix, k_suffix, scale)
    S, Hq, D = q.shape
    with torch.cuda.device(q.device):
        out = _output(out, (S, Hq, D), q.device, "out")
        lse = _output(lse, (S, Hq), q.device, "lse")
        n = ctypes.c_size_t(0)
        _check(lib.attn_bifurcated_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
               "attn_bifurcated_workspace_bytes")
        ws = _workspace(n.value, q.device, workspace)
        nbytes = 0 if ws is None else ws.numel() * ws.element_size()
        _check(lib.attn_decode_bifurcated(ctypes.byref(desc), _ptr(q), _ptr(k_prefix),
                                          _ptr(v_prefix), _ptr(k_suffix), _ptr(v_suffix),
                                          _ptr(out), _ptr(lse), _ptr(ws), nbytes,
                                          _stream_ptr(q.device)), "attn_decode_bifurcated")
    return out, lse


class BifurcatedCall:
    """attn_decode_bifurcated prepared once for fixed tensors: descriptor,
    outputs and workspace are set up here, and ``run()`` is only the C call
    (for repeated calls, where the per-call Python work would otherwise be
    comparable to the GPU time of a small batch)."""

    def __init__(self, q, k_prefix, v_prefix, k_suffix, v_suffix, *, scale=None):
        torch = _torch()
        self.lib = load_library()
        _check_tensors(q, k_prefix, v_prefix, k_suffix, v_suffix)
        if v_prefix.shape != k_prefix.shape or v_suffix.shape != k_suffix.shape:
            raise ValueError("v tensors must match k tensors")
        self.desc = bifurcated_desc(q, k_prefix, k_suffix, scale)
        S, Hq, D = q.shape
        with torch.cuda.device(q.device):
            self.out = torch.empty((S, Hq, D), dtype=torch.float32, device=q.device)
            self.lse = torch.empty((S, Hq), dtype=torch.float32, device=q.device)
            n = ctypes.c_size_t(0)
            _check(self.lib.attn_bifurcated_workspace_bytes(ctypes.byref(self.desc), ctypes.byref(n)),
                   "attn_bifurcated_workspace_bytes")
            self.ws = _workspace(n.value, q.device, None)
            self.stream = _stream_ptr(q.device)
        self.nbytes = 0 if self.ws is None else self.ws.numel()
        self.args = [ctypes.byref(self.desc)] + [_ptr(t) for t in (q, k_prefix, v_prefix, k_suffix,
                                                                   v_suffix, self.out, self.lse)]
        self.args += [_ptr(self.ws), self.nbytes, self.stream]

    def run(self):
        _check(self.lib.attn_decode_bifurcated(*self.args), "attn_decode_bifurcated")
        return self.out, self.lse


def anchor_desc(q, k_anchor, k_blocks, scale=None) -> AttnAnchorDesc:
    if q.dim() != 4 or k_anchor.dim() != 3 or k_blocks.dim() != 4:
        raise ValueError("q [N,Lb,Hq,D], k_anchor [Hkv,A,D], k_blocks [N,Hkv,Lb,D]")
    N, Lb, Hq, D = q.shape
    Hkv, A, Da = k_anchor.shape
    if tuple(k_blocks.shape) != (N, Hkv, Lb, D) or Da != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k_anchor{tuple(k_anchor.shape)} "
                         f"k_blocks{tuple(k_blocks.shape)}")
    d = AttnAnchorDesc()
    d.num_blocks, d.block_len, d.num_q_heads, d.num_kv_heads, d.head_dim = N, Lb, Hq, Hkv, D
    d.anchor_len = A
    d.scale = (1.0 / math.sqrt(D)) if scale is None else scale
    d.dtype = _dtype_code(q)
    return d


def prefill_anchor(q, k_anchor, v_anchor, k_blocks, v_blocks, *, scale: Optional[float] = None,
                   out=None, lse=None, workspace=None):
    """Context encoding with an anchor block: returns (O float32 [N,Lb,Hq,D],
    lse float32 [N,Lb,Hq]); block b's query i sees the whole anchor and its
    block's keys t <= i."""
    torch = _torch()
    lib = load_library()
    _check_tensors(q, k_anchor, v_anchor, k_blocks, v_blocks)
    if v_anchor.shape != k_anchor.shape or v_blocks.shape != k_blocks.shape:
        raise ValueError("v tensors must match k tensors")
    desc = anchor_desc(q, k_anchor, k_blocks, scale)
    N, Lb, Hq, D = q.shape
    with torch.cuda.device(q.device):
        out = _output(out, (N, Lb, Hq, D), q.device, "out")
        lse = _output(lse, (N, Lb, Hq), q.device, "lse")
        n = ctypes.c_size_t(0)
        _check(lib.attn_anchor_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
               "attn_anchor_workspace_bytes")
        ws = _workspace(n.value, q.device, workspace)
        nbytes = 0 if ws is None else ws.numel() * ws.element_size()
        _check(lib.attn_prefill_anchor(ctypes.byref(desc), _ptr(q), _ptr(k_anchor), _ptr(v_anchor),
                                       _ptr(k_blocks), _ptr(v_blocks), _ptr(out), _ptr(lse),
                                       _ptr(ws), nbytes, _stream_ptr(q.device)),
               "attn_prefill_anchor")
    return out, lse


def testing_prefill_anchor_unfused(q, k_anchor, v_anchor, k_blocks, v_blocks, *,
                                   scale: Optional[float] = None):
    """prefill_anchor forced onto its three-launch path (test build only)."""
    torch = _torch()
    lib = load_testing_library()
    _check_tensors(q, k_anchor, v_anchor, k_blocks, v_blocks)
    desc = anchor_desc(q, k_anchor, k_blocks, scale)
    N, Lb, Hq, D = q.shape
    with torch.cuda.device(q.device):
        out = _output(None, (N, Lb, Hq, D), q.device, "out")
        lse = _output(None, (N, Lb, Hq), q.device, "lse")
        n = ctypes.c_size_t(0)
        _check(load_library().attn_anchor_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
               "attn_anchor_workspace_bytes")
        ws = _workspace(n.value, q.device, None)
        nbytes = 0 if ws is None else ws.numel() * ws.element_size()
        _check(lib.attn_testing_prefill_anchor_unfused(
            ctypes.byref(desc), _ptr(q), _ptr(k_anchor), _ptr(v_anchor), _ptr(k_blocks),
            _ptr(v_blocks), _ptr(out), _ptr(lse), _ptr(ws), nbytes, _stream_ptr(q.device)),
            "attn_testing_prefill_anchor_unfused")
    return out, lse
