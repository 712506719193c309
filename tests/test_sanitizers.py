"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the C oracle with its pins (tests/sanitize/oracle_asan.c) and the C-ABI
layer's validation, workspace sizing and launch descriptors with the kernel
dispatchers stubbed out (tests/sanitize/api_asan.cpp).  Any sanitizer report
aborts the program (-fno-sanitize-recover), so a clean exit is the check."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd_build, exe):
    out = subprocess.run(cmd_build, capture_output=True, text=True, cwd=ROOT)
    assert out.returncode == 0, out.stderr[-4000:]
    res = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    print(res.stdout)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr
    assert "all ok" in res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-std=c99", "-fopenmp"] + FLAGS +
         ["-o", exe, os.path.join(SAN, "oracle_asan.c"), os.path.join(ROOT, "oracle", "gsa_oracle.c"),
          "-lm"], exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_abi_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_asan")
    _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"] + FLAGS +
         ["-o", exe, os.path.join(SAN, "api_asan.cpp"),
          os.path.join(ROOT, "slot_memory_sequence_amd", "csrc", "api.cpp")], exe)
