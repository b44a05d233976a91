"""The C-ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): builds the sanitizer test library (host code instrumented, see
block_sparse_attention_losa_amd/build.py) and runs the C-ABI checks of
tests/test_abi.py against it in a child process with the sanitizer runtime
preloaded.  Any sanitizer report fails the run: UBSan is built not to
recover, and ASan reports (which abort) go to a log that must stay empty."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

from block_sparse_attention_losa_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_abi_checks_are_clean_under_host_sanitizers(tmp_path):
    lib = build.build_sanitized()
    runtime = build.sanitizer_runtime()
    log = str(tmp_path / "sanitizer")
    env = dict(os.environ)
    env.update({
        "LOSA_LIBRARY": lib,
        "LD_PRELOAD": runtime,
        # the interpreter itself is not instrumented: its own allocations are
        # not leak-checked, only the library's accesses and its undefined
        # behaviour are
        "ASAN_OPTIONS": f"detect_leaks=0:log_path={log}",
        "UBSAN_OPTIONS": f"print_stacktrace=1:log_path={log}",
    })
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = sorted(glob.glob(log + "*"))
    text = "".join(open(p).read() for p in reports)
    assert res.returncode == 0 and not reports, (res.stdout[-3000:], res.stderr[-3000:], text)
    assert " passed" in res.stdout
