"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, gcc): the oracle pins (tests/test_oracle_pins.py) run against that
build in a child process (ORACLE_LIB names it; the sanitizer runtime is
preloaded, as the Python interpreter itself is not instrumented).  Any
out-of-bounds access, use after free or undefined operation in the oracle
aborts the child, and the test fails."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], stdout=subprocess.PIPE, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no AddressSanitizer runtime for gcc here")
    with tempfile.TemporaryDirectory() as tmp:
        so = os.path.join(tmp, "liboracle_san.so")
        subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared",
                               "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                               "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "oracle"),
                               "-o", so, SRC, "-lm"])
        env = dict(os.environ, ORACLE_LIB=so, LD_PRELOAD=asan,
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        p = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                           cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                           text=True, timeout=900)
    assert p.returncode == 0, p.stdout[-4000:]
    assert "passed" in p.stdout
