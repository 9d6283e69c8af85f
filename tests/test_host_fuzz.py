"""Randomized host test of the copy planner and the block pool under
AddressSanitizer and UndefinedBehaviorSanitizer (host code only; no GPU).

Builds tests/host_fuzz/fuzz_host.cpp with the library's pool.cpp and
copy_plan.cpp into a temporary directory and runs it: every plan must equal
the moves applied one by one in pkv_order_moves order ("KV Cache Design —
cells, format, sessions", section 2), and every pool history must keep each
block's reference count equal to the table entries naming it; any
out-of-bounds access or undefined behaviour aborts the run.
"""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_table_amd", "csrc")


def _hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


def test_host_planners_under_sanitizers():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "fuzz_host")
        cmd = [hipcc, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all", "-fno-gpu-sanitize",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip",
               os.path.join(CSRC, "pool.cpp"), os.path.join(CSRC, "copy_plan.cpp"),
               os.path.join(ROOT, "tests", "host_fuzz", "fuzz_host.cpp"), "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        # the sanitizer runtime need not come first in the load order
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe, "5000", "500"], capture_output=True, text=True, env=env, timeout=600)
        assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
        assert "copy plan: 5000 cases ok" in r.stdout and "pool: 500 histories ok" in r.stdout
