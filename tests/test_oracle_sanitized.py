"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer:
oracle.c is rebuilt with -fsanitize=address,undefined (host code only; the
GPU library is not involved) and tests/test_oracle.py runs against that build
in a child process, with the ASan runtime preloaded into the child (Python
itself is not instrumented).  Any out-of-bounds access, use after free or
undefined behaviour in the oracle aborts the child and fails this test."""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _libasan():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                           check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_sanitizers(tmp_path):
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc's libasan is not installed")
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a preload is already set for this process; the sanitizer run needs its own")
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan,
        "TERNARY_ORACLE_LIB": lib,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle.py"), "-q", "-x",
                        "-m", "not gpu", "-p", "no:cacheprovider"],
                       cwd=os.path.dirname(HERE), env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "error" not in r.stdout.lower().split("passed")[-1], tail
