"""The C ABI's argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: tests/validate_sanitized.cpp calls
every check with extreme arguments (int32 and int64 limits, negatives,
misaligned and null pointers) and checks the statuses; a signed overflow or
any other undefined behaviour aborts it.  Host code only (g++, no HIP)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_checks_have_no_undefined_behaviour(tmp_path):
    exe = tmp_path / "validate_sanitized"
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
         "-I", os.path.join(ROOT, "fp8_kv_cache_slot_amd", "csrc"),
         os.path.join(ROOT, "tests", "validate_sanitized.cpp"), "-o", str(exe)],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
