"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/oracle_sanitized.cpp builds oracle/oracle.cpp with both sanitizers and
calls every oracle entry on small inputs in buffers of exactly the documented
size, with the documented edge cases (skipped and out-of-range slots, invalid
pages, sequence lengths past the block table, rows past the output, partial
and zero rotary, both pairings and dtypes), and every number-format routine
over its whole input range.  An out-of-bounds access, a signed overflow or
any other undefined behaviour in the oracle aborts it.  Host code only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_has_no_undefined_behaviour(tmp_path):
    exe = tmp_path / "oracle_sanitized"
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "oracle"),
         os.path.join(ROOT, "tests", "oracle_sanitized.cpp"),
         os.path.join(ROOT, "oracle", "oracle.cpp"), "-o", str(exe)],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
