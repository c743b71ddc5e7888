"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_driver.c compiles the oracle's source into a program that
calls every entry point over small ragged tensors in every mode (formats,
tensor/block scales, POW2/AMAX, fp32/bf16 master, coupled L2, delayed scaling,
stochastic rounding, the other update-order reading, the fp32-moment mode, the
gradient sums and the loss-scaler decision).  Host code only, built with gcc."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    build = subprocess.run(
        ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
         "-ffp-contract=off", "-o", exe, os.path.join(HERE, "oracle_sanitize_driver.c"), "-lm"],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1"))
    assert run.returncode == 0, run.stderr[-4000:]
    assert "oracle driver done" in run.stdout
    assert "runtime error" not in run.stderr and "Sanitizer" not in run.stderr, run.stderr[-4000:]
