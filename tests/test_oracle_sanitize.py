"""The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(g++, host code only), driven through every entry point on tiny layers of
each storage format and through its argument checks
(tests/oracle_sanitize_main.cpp).  Any out-of-bounds access, use after free,
leak, signed overflow, bad shift or misaligned load fails the test."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE = os.path.join(os.path.dirname(HERE), "oracle")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer"]
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fopenmp", "-ffp-contract=off", *san,
                    "-I", ORACLE, "-o", str(exe), os.path.join(ORACLE, "oracle.cpp"),
                    os.path.join(HERE, "oracle_sanitize_main.cpp")], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitizer run ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
