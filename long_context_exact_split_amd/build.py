"""Build ``libattn_decode.so`` for gfx950 with hipcc (in-tree).

Every HIP/C++ source under ``csrc/`` is compiled to an object in ``_build/``
(in parallel), then linked into the shared library next to this file.  The
test build ``libattn_decode_testing.so`` links the same objects plus the
test-only hooks under ``csrc/testing/``; the product library holds none of
them.  ``libattn_decode_stamps.so`` is the product with its decode split
kernels built to time every workgroup (bench.py --wg-stamps), and
``libhbm_probe.so`` holds the HBM reference kernels.  Symbols are hidden
unless the public headers mark them ATTN_API.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libattn_decode.so"
TESTING_LIB_NAME = "libattn_decode_testing.so"
PROBE_NAME = "libhbm_probe.so"  # HBM read-stream / copy reference kernels
# The product library with the decode split kernels (vector-ALU and 32-row
# matrix-core) and the one-launch shared-prefix kernel built to record each
# workgroup's start and end clocks and XCD
# (csrc/probe/wg_stamps.h); loaded only by the bench's --wg-stamps
# measurement.  Each stamped source has its own stamp array and read-back.
STAMPS_LIB_NAME = "libattn_decode_stamps.so"
STAMPED_SOURCES = ("split_kv_valu.hip", "split_kv_mfma.hip", "split_kv_bifurcated.hip")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
          "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]
# Packed fp32 VALU ops are kept out of the generated code.
HIP_ONLY = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Optional kernel tuning parameters (e.g. "-DATTN_SPLIT_KT_SMALL=16"); the
# defaults in the sources are the measured choices.
DEFINES = os.environ.get("ATTN_BUILD_DEFINES", "").split()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool, extra=(), suffix: str = "") -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + suffix + ".o")
    cmd = [hipcc(), "-c", src, "-o", obj] + COMMON + DEFINES + list(extra)
    if src.endswith(".hip"):
        cmd = [hipcc(), "-x", "hip", "-c", src, "-o", obj] + HIP_ONLY + COMMON + DEFINES + \
            list(extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    return obj


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def testing_sources():
    return sorted(glob.glob(os.path.join(CSRC, "testing", "*.cpp")))


def _link(objs, name, verbose, out_dir=PKG):
    out = os.path.join(out_dir, name)
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, out_dir: str = PKG, build_dir: str = BUILD) -> str:
    """Compile every source and link the library; returns its path."""
    global BUILD
    BUILD = build_dir
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    tsrcs = testing_sources()
    probe = os.path.join(CSRC, "probe", "hbm_probe.hip")
    jobs = [(s, (), "") for s in srcs + tsrcs + [probe]]
    jobs += [(os.path.join(CSRC, name), ("-DATTN_WG_STAMPS",), ".stamps")
             for name in STAMPED_SOURCES]
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1], j[2]), jobs))
    lib_objs, test_objs = objs[:len(srcs)], objs[len(srcs):len(srcs) + len(tsrcs)]
    probe_obj = objs[len(srcs) + len(tsrcs)]
    stamped = dict(zip(STAMPED_SOURCES, objs[len(srcs) + len(tsrcs) + 1:]))
    _link([probe_obj], PROBE_NAME, verbose, out_dir)
    _link(lib_objs + test_objs, TESTING_LIB_NAME, verbose, out_dir)
    _link([stamped.get(os.path.basename(s), o) for s, o in zip(srcs, lib_objs)],
          STAMPS_LIB_NAME, verbose, out_dir)
    return _link(lib_objs, LIB_NAME, verbose, out_dir)


if __name__ == "__main__":
    print(build(verbose=True))
