"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

plan.cpp (validation, partition and plans, including work_map.h's layout
arithmetic) and the test hooks are compiled with g++ and
-fsanitize=address,undefined into a host-only library (no HIP code).  A
child pytest then drives it through the partition, anchor-path, host-check and
shared-prefix launch-form tests (hypothesis shapes, ragged and causal layouts,
and the extreme shapes with 2^16 rows per KV head and 2^31 - 2^16 tokens),
with the sanitizer runtime preloaded and every report fatal.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_exact_split_amd", "csrc")


def _runtime(name):
    path = subprocess.run(["g++", "-print-file-name=" + name], capture_output=True, text=True,
                          check=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    if not shutil.which("g++"):
        pytest.skip("g++ not available")
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("AddressSanitizer runtime not available")
    lib = tmp_path / "libattn_host_sanitized.so"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
           "-fvisibility=hidden", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "testing", "testing_hooks.cpp"), "-o", str(lib)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ)
    env.update(ATTN_TESTING_LIB=str(lib), LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               HYPOTHESIS_STORAGE_DIRECTORY=str(tmp_path / "hyp"))
    tests = [os.path.join(ROOT, "tests", t) for t in
             ("test_partition.py", "test_anchor_fusion.py", "test_host_checks.py",
              "test_bifurcated_form.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    # -s: a report goes to the terminal, not into pytest's capture, before the
    # runtime ends the process
    assert r.returncode == 0, out[:6000]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
