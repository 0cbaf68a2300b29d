"""The oracle's pins once more with the oracle built under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

A child pytest runs the oracle's own test files (the golden cases, closed forms,
identities, finite differences and the planted mistakes, whose broken copies are built
with the same sanitizers) against a sanitized build of oracle/wkv_oracle.c, with gcc's
libasan preloaded. Any out-of-bounds access, use of freed memory, signed overflow,
misaligned access or other undefined behaviour aborts the child with the sanitizer's
report, and this test fails with it.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PINS = ["test_oracle_forward.py", "test_oracle_backward.py", "test_oracle_decode.py",
        "test_oracle_state.py", "test_oracle_gate.py", "test_golden_regression.py",
        "test_oracle_mutations.py"]


def _runtime(name):
    try:
        path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                              text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's libasan is not installed")
    env = dict(os.environ)
    env.update(WKV_ORACLE_SANITIZE="1", LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
    cmd += [os.path.join(HERE, f) for f in PINS]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
