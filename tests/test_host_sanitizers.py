"""The host half of the C ABI (coda_host.cpp: workspace sizes, argument validation, status strings)
built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and driven through valid and
invalid arguments, including extreme sizes and enum fields holding arbitrary ints (CPU only; the
HIP kernels are not part of that compilation)."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_gemm_epilogue_res_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "validate_main.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_validation_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "validate")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               os.path.join(CSRC, "coda_host.cpp"), DRIVER, "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        env.pop("LD_PRELOAD", None)
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
        assert "ok" in r.stdout
