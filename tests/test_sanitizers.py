"""AddressSanitizer and UndefinedBehaviorSanitizer runs of the host code (no
GPU): the library's canonical -> planar repack (pack.cpp, built with g++) and
the CPU oracle (qgemm_oracle.c, built with gcc), each driven over every codec
by a small driver under tests/sanitize/.  The pages report their host code
leak-free (releases page v0.2.3); an out-of-bounds access, a leak or undefined
behaviour aborts the driver here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-Wall", "-Wextra", "-Werror"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _build_and_run(tmp_path, compiler, sources, extra):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not available")
    exe = str(tmp_path / "driver")
    subprocess.run([compiler, *SAN, *extra, *sources, "-o", exe], check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


def test_pack_host_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "g++", [os.path.join(ROOT, "tests", "sanitize", "pack_driver.cpp"),
                                           os.path.join(ROOT, "quantized_prefill_gemm_codec_amd", "csrc", "pack.cpp")],
                         ["-std=c++17", "-I" + os.path.join(ROOT, "include")])
    assert "all calls returned the expected status" in out


def test_oracle_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "gcc", [os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                                           os.path.join(ROOT, "oracle", "qgemm_oracle.c")],
                         ["-std=c11", "-ffp-contract=off", "-Wno-unknown-pragmas", "-lm"])
    assert "all calls returned the expected status" in out
