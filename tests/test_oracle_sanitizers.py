"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code, gcc).

oracle/sanitize_driver.c calls every entry point of oracle/pkv_oracle.c on small inputs,
error paths included, and checks a few results; built with both sanitizers (and leak
detection), any out-of-bounds access, use after free, leak or undefined operation makes the
run fail.  Once without OpenMP (the loops as plain serial C) and once with it."""
import os
import shutil
import subprocess

import pytest

from oracle.build import SRC

DRIVER = os.path.join(os.path.dirname(SRC), "sanitize_driver.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("openmp", [False, True], ids=["serial", "openmp"])
def test_oracle_under_asan_and_ubsan(tmp_path, openmp):
    exe = tmp_path / "sanitize_driver"
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-Wall", DRIVER, SRC, "-o", str(exe), "-lm"]
    if openmp:
        cmd.insert(1, "-fopenmp")
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               OMP_NUM_THREADS="4")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "sanitize_driver: 0 failure(s)" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
