"""The host side of the library under AddressSanitizer and
UndefinedBehaviorSanitizer: the sources' host code is built sanitized into a
separate library (build.build_host_sanitized), and the C-ABI tests and the
schedule tests run against it in a child python with the sanitizer runtime
preloaded.  Any report (out-of-bounds access, use after free, signed
overflow, invalid enum load, ...) fails the test.  No GPU is used: every
call these tests make either stays on the host or fails its argument checks
before the HIP runtime is reached."""

import glob
import os
import subprocess
import sys

import pytest

from long_context_exact_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized_lib():
    try:
        return B.build_host_sanitized()
    except (OSError, RuntimeError) as e:  # no hipcc here
        pytest.skip(f"cannot build the sanitized library: {e}")


def test_abi_and_schedules_clean_under_asan_ubsan(sanitized_lib, tmp_path):
    rt = B.sanitizer_runtime()
    assert os.path.exists(rt), rt
    logs = tmp_path / "san"
    env = dict(os.environ,
               LD_PRELOAD=rt, DFA_LIBRARY=sanitized_lib,
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={logs}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={logs}")
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
         os.path.join(ROOT, "tests", "test_abi.py"),
         os.path.join(ROOT, "tests", "test_oracle_schedule.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = sorted(glob.glob(str(logs) + "*"))
    text = "".join(open(f).read() for f in reports)
    assert not reports, f"sanitizer reports:\n{text[:4000]}"
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert " passed" in res.stdout
