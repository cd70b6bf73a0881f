"""The oracle's pins, run once against an AddressSanitizer + UndefinedBehavior-
Sanitizer build of oracle.c (host only, no GPU): any out-of-bounds access, use
after free, signed overflow, misaligned load or other undefined behaviour in the
C oracle stops the child process with a report, and fails this test."""

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["test_oracle.py", "test_oracle_append.py", "test_oracle_chunk.py", "test_oracle_backward.py"]


def _libasan():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_libasan() is None, reason="gcc has no AddressSanitizer runtime here")
def test_oracle_pins_clean_under_asan_ubsan(tmp_path):
    lib = oracle.build(sanitize=True, out=str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=_libasan(), OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    files = [os.path.join(ROOT, "tests", f) for f in PIN_FILES]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *files], env=env, capture_output=True, text=True,
                       timeout=900, cwd=ROOT)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert "AddressSanitizer" not in report and "runtime error" not in report, report
    assert r.returncode == 0, report
    assert " passed" in r.stdout, report


@pytest.mark.skipif(_libasan() is None, reason="gcc has no AddressSanitizer runtime here")
def test_sanitizer_harness_reports_a_planted_overflow(tmp_path):
    """Control for the run above: with the same flags and preload, a read one
    element past a heap array in a tiny C library is reported and stops the child."""
    src = tmp_path / "overflow.c"
    src.write_text("#include <stdlib.h>\n"
                   "double read_past(int n) { double *a = malloc(n * sizeof(double));\n"
                   "  for (int i = 0; i < n; ++i) a[i] = i;\n"
                   "  double s = a[n]; free(a); return s; }\n")
    lib = tmp_path / "liboverflow.so"
    subprocess.run(["gcc", *oracle.SANITIZE_FLAGS, "-fPIC", "-shared", str(src), "-o", str(lib)], check=True)
    code = ("import ctypes; f = ctypes.CDLL(%r).read_past; f.restype = ctypes.c_double; "
            "print(f(8))" % str(lib))
    env = dict(os.environ, LD_PRELOAD=_libasan(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
