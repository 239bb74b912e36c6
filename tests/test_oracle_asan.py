"""Host sanitizers on the float64 oracle: oracle/la_oracle.c and the driver
tests/asan/oracle_driver.c built with gcc -fsanitize=address,undefined and run
as an executable (no Python process loads the instrumented code).  The
driver calls every oracle routine on empty, single-token and ragged shapes
with buffers of exactly the size each routine may touch, so any read or write
past a buffer, any use after free and any undefined arithmetic stops the run.
A harness check first shows that the same build flags do stop an
off-by-one write."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
FLAGS = ["-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined", "-Wno-unknown-pragmas"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed for the sanitizer build")


def _build(tmp_path, sources, name):
    exe = str(tmp_path / name)
    res = subprocess.run(["gcc", *FLAGS, "-o", exe, *sources, "-lm"], capture_output=True, text=True)
    if res.returncode != 0 and "asan" in (res.stderr or "").lower():
        pytest.skip("the AddressSanitizer runtime is not installed")
    assert res.returncode == 0, res.stderr
    return exe


def test_sanitizer_catches_an_overflow(tmp_path):
    src = tmp_path / "overflow.c"
    src.write_text("#include <stdlib.h>\nint main(void) {\n  double *p = malloc(4 * sizeof(double));\n"
                   "  for (int i = 0; i <= 4; ++i) p[i] = i;\n  free(p);\n  return 0;\n}\n")
    exe = _build(tmp_path, [str(src)], "overflow")
    res = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=60)
    # stopped by the address checks or, first, by the undefined-behaviour object-size check
    assert res.returncode != 0 and ("AddressSanitizer" in res.stderr or "runtime error" in res.stderr), res.stderr


def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = _build(tmp_path, [os.path.join(ROOT, "oracle", "la_oracle.c"), os.path.join(HERE, "asan", "oracle_driver.c")],
                 "oracle_driver")
    res = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ok (0 failures)" in res.stdout
    assert "runtime error" not in res.stderr and "Sanitizer" not in res.stderr, res.stderr
