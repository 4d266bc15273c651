"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers (tests/sanitize/) are built with -fsanitize=address,undefined and
run: the oracle's every entry point over all head sizes, rotations, groups
and code widths; and the C ABI's validation and argument marshalling
(csrc/api.cpp, with the kernel dispatchers stubbed), including sizes at the
int64 edges.  Any sanitizer report fails the run (no recovery)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, cwd=None):
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=cwd, timeout=300)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-ffp-contract=off"] + SAN +
         [os.path.join(ROOT, "oracle", "srftq_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          "-o", exe, "-lm"])
    assert "oracle driver: ok" in _run([exe])


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_abi_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    csrc = os.path.join(ROOT, "kv_cache_quantization_srft_amd", "csrc")
    _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
          "-I", csrc] + SAN + [os.path.join(csrc, "api.cpp"), os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"),
                               "-o", exe])
    assert "abi driver: ok" in _run([exe])
