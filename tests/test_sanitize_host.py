"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The planner is a few thousand lines of index arithmetic over fixed-size mode
arrays (the canonical shard, the kernels' mode tables, the 2^31 and 2^58
bounds); the entry points validate and cache plans across threads.  This
builds the library with both sanitizers on its host code and reruns the CPU
tests that drive it -- exports, every decline, plan choices, the bank
models, thread safety, the in-place unit order, the kernels' CPU index
models and the brute-force planner cross-checks -- in a child process that
loads that build.  Any sanitizer report fails the child and this test.
No GPU is used: nothing launches a kernel."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

from tensor_layout_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_abi_cpu.py", "tests/test_plan_bruteforce.py", "tests/test_rec_model.py",
          "tests/test_etile_model.py", "tests/test_etile_vec_model.py", "tests/test_oracle_swizzle_pins.py",
          "tests/test_plan_oracle.py"]


@pytest.mark.skipif(not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import sanitize_build
    lib = sanitize_build.build_sanitized(str(tmp_path))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the build is not instrumented"
    # Reports go to files: pytest captures the child's stderr, and a halted
    # process never prints what it captured.
    logs = tmp_path / "reports"
    logs.mkdir()
    env = dict(os.environ, TPL_LIBRARY=lib, LD_PRELOAD=sanitize_build.runtime(),
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={logs}/asan",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={logs}/ubsan")
    # four worker processes (each inherits the preloaded runtime and the
    # report paths, which get the process id appended)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                          "-n", "4"] + SUITES, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    reports = "".join(f.read_text()[:3000] for f in sorted(logs.iterdir()))
    assert not reports, reports
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
