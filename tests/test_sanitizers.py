"""The CPU oracle and the library's host-side stream validator built with
AddressSanitizer and UndefinedBehaviorSanitizer (gcc / g++, host code only)
and run on small seeded inputs of every format, including corrupted streams.
Any out-of-bounds access, leak or undefined behaviour fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout}\n{p.stderr}"
    return p.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-std=c11", *SAN, "-I", os.path.join(ROOT, "oracle"), "-o", exe,
         os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "cass_oracle.c"), "-lm"])
    assert "oracle driver ok" in run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="needs g++")
def test_validator_under_sanitizers(tmp_path):
    exe = str(tmp_path / "validate_driver")
    obj = str(tmp_path / "cass_oracle.o")
    run(["gcc", "-std=c11", *SAN, "-c", "-o", obj, os.path.join(ROOT, "oracle", "cass_oracle.c")])
    run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
         "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "oracle"), "-o", exe,
         os.path.join(HERE, "validate_driver.cpp"),
         os.path.join(ROOT, "bit_level_weight_amd", "csrc", "validate.cpp"), obj, "-lm"])
    assert "validate driver ok" in run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
