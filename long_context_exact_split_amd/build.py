"""Build ``libattn_decode.so`` for gfx950 with hipcc (in-tree).

Every HIP/C++ source under ``csrc/`` is compiled to an object in ``_build/``
(in parallel), then linked into the shared library next to this file.
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
PROBE_NAME = "libhbm_probe.so"  # HBM read-stream / copy reference kernels
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", INCLUDE, "-I", CSRC]
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


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-c", src, "-o", obj] + COMMON + DEFINES
    if src.endswith(".hip"):
        cmd = [hipcc(), "-x", "hip", "-c", src, "-o", obj] + HIP_ONLY + COMMON + DEFINES
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    return obj


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


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
    probe = os.path.join(CSRC, "probe", "hbm_probe.hip")
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs + [probe]))
    _link(objs[-1:], PROBE_NAME, verbose, out_dir)
    return _link(objs[:-1], LIB_NAME, verbose, out_dir)


if __name__ == "__main__":
    print(build(verbose=True))
