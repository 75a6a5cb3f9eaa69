"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): tests/sanitize/driver.cpp drives the oracle, the library's text-form
parsers and its hash-table placement on seeded random tables and inputs,
error paths included; any sanitizer report or failed check fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def test_host_code_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("gcc/g++ not available")
    obj = tmp_path / "oracle.o"
    exe = tmp_path / "driver"
    subprocess.run(["gcc", "-std=c11", *SAN, "-c", os.path.join(ROOT, "oracle", "bpe_oracle.c"),
                    "-o", str(obj)], check=True)
    csrc = os.path.join(ROOT, "byte_level_bpe_pretokenize_amd", "csrc")
    # the tables' source includes the HIP runtime header for its layouts; it
    # makes no HIP call, so the host compiler builds it without the runtime
    subprocess.run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    os.path.join(ROOT, "tests", "sanitize", "driver.cpp"),
                    os.path.join(csrc, "bpe_text.cpp"), os.path.join(csrc, "bpe_tables.cpp"),
                    str(obj), "-o", str(exe)], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "passed" in r.stdout
