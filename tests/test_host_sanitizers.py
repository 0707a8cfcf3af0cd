"""The host C++ of the library (allocator, prefix registry, cascade planner)
under AddressSanitizer and UndefinedBehaviorSanitizer, CPU only.

``host_stress.cpp`` drives the C ABI with random operations and checks,
after every step, invariants that hold for any history: reference counts
equal the table and registry entries that point at each block, the free
stack holds exactly the unreferenced blocks, and every planned work item
lies inside its sequence's context and the plan's bounds.  It is built here
with g++ from the same sources as ``libpa.so``'s host objects.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_198_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_stress")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined",
           "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host_stress.cpp"),
           os.path.join(CSRC, "pa_alloc.cpp"), os.path.join(CSRC, "pa_cascade.cpp"),
           "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([exe, "6"], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "host stress ok" in run.stdout
