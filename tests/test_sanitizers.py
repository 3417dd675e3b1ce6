"""The oracle and the seeded input generator built with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only) and driven through every entry
point on small inputs by oracle/sanitize_driver.cpp; any invalid access,
leak or undefined operation fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs gcc/g++")
def test_oracle_and_datagen_under_asan_ubsan(tmp_path):
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-g", "-O1"]
    dg_obj = tmp_path / "philox_normal.o"
    subprocess.run(["gcc", "-std=c11", *san, "-c", os.path.join(ROOT, "datagen", "philox_normal.c"),
                    "-o", str(dg_obj)], check=True)
    exe = tmp_path / "sanitize_driver"
    subprocess.run(["g++", "-std=c++17", *san, "-fopenmp",
                    os.path.join(ROOT, "oracle", "sanitize_driver.cpp"),
                    os.path.join(ROOT, "oracle", "moe_oracle.cpp"), str(dg_obj), "-o", str(exe),
                    "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([str(exe)], env=env, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ok" in res.stdout
