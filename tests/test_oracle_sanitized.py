"""The oracle's pins again, on a build of the oracle with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, host code only): an out-of-bounds access, a
use after free, a signed overflow or a misaligned load anywhere on the pinned
paths aborts the child process and fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib(name):
    try:
        p = subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = _lib("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    so = str(tmp_path / "libspkv_oracle_san.so")
    subprocess.check_call([
        "gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-Wall", "-Wextra", "-fno-omit-frame-pointer",
        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared", "-fPIC",
        "-o", so, os.path.join(ROOT, "oracle", "spkv_oracle.c"), "-lm"])
    env = dict(os.environ)
    env.update({
        "SPKV_ORACLE_LIB": so,
        "LD_PRELOAD": asan,
        # the interpreter's own allocations are not the oracle's: no leak report
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:allocator_may_return_null=0",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "OMP_NUM_THREADS": "4",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
