"""The host bookkeeping of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer: the
mock-launcher tests and the log-based filter's planner tests, run in a child process against a
sanitized build of the host code (g++, CPU only; no device code is built or run)."""
import os
import subprocess
import sys

import pytest

from packed_cache_decode_block_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    r = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_host_logic_under_asan_and_ubsan():
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("no AddressSanitizer runtime for g++")
    build_lib.build_mock(sanitize=True)
    env = dict(os.environ, BGTQ_SANITIZED_MOCK="1", LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_host_mock.py", "tests/test_logquant_plan_cpu.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout[-4000:] + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
