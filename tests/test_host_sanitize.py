"""The host table builders (csrc/host.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/host_sanitize_driver.cpp, compiled with g++ beside host.cpp (host code only, no device
code), builds random attention tables (with and without shared-prefix groups) and random GEMM
tables, first into undersized buffers (which must report PA_ERR_CAPACITY without writing past
them) and then into exact-size ones. Any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_table_builders_under_sanitizers(tmp_path):
    exe = str(tmp_path / "drive")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"),
                    os.path.join(ROOT, "paged_variable_length_amd", "csrc", "host.cpp"),
                    "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "800", "600"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok 1400," in r.stdout, r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
