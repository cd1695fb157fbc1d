"""The C ABI's argument validation built on the host alone, under
AddressSanitizer and UndefinedBehaviorSanitizer.

fa_validate.cpp holds every precondition check of include/flash_attn.h and
the normalisation of the arguments; it has no HIP dependency. This test
compiles it with g++ together with tests/host/validate_driver.cpp (the
invalid-argument table, the normalised parameters of valid calls, and a
deterministic fuzz over extreme sizes and addresses) and requires a clean run:
any sanitizer report aborts the program.
"""
from __future__ import annotations

import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_validation_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "validate_driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", str(ROOT / "include"),
           str(ROOT / "io_aware_tiled_flash_amd/csrc/fa_validate.cpp"),
           str(ROOT / "tests/host/validate_driver.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                         env={"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                              "UBSAN_OPTIONS": "print_stacktrace=1", "PATH": "/usr/bin:/bin"})
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ALL OK" in res.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
