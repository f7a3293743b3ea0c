"""The fp64 CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/gmm_oracle.c is built with gcc together with a small driver
(tests/oracle_sanitize_driver.c) that calls every entry point on seeded
inputs and edge cases; the run must exit 0 with no sanitizer report. One
build is single-threaded with ASan + UBSan, one multi-threaded (OpenMP) with
UBSan. Host code only.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = [os.path.join(HERE, "oracle_sanitize_driver.c"), os.path.join(ROOT, "oracle", "gmm_oracle.c")]


@pytest.mark.parametrize("flags", [
    ["-fsanitize=address,undefined"],
    ["-fopenmp", "-fsanitize=undefined"],
], ids=["asan+ubsan", "ubsan+openmp"])
def test_oracle_under_sanitizers(tmp_path, flags):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer",
                    "-fno-sanitize-recover=all", *flags, *SRC, "-o", exe, "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok", r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr
