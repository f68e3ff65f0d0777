"""The host-side C++ of the C ABI (argument checks and sizing) and the C
oracle, each built on its own with AddressSanitizer and
UndefinedBehaviorSanitizer and driven through its edge cases
(tests/native/*): an out-of-bounds access, a signed overflow or another
undefined operation aborts the driver.  Host code only (g++ / gcc): the HIP
kernels are not built here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiled_attention_transformer_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _build_and_run(cmd, exe):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "0 failed" in r.stdout
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks_driver")
    out = _build_and_run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__",
                          "-I/opt/rocm/include", "-I" + CSRC,
                          os.path.join(NATIVE, "host_checks_driver.cpp"),
                          os.path.join(CSRC, "host_checks.cpp"), "-o", exe], exe)
    print(out)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    out = _build_and_run(["gcc", "-std=c11", "-fopenmp", *SAN,
                          os.path.join(NATIVE, "oracle_driver.c"),
                          os.path.join(ROOT, "oracle", "oracle_cpu.c"), "-lm", "-o", exe], exe)
    print(out)
