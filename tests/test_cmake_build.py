"""The CMake build (CMakeLists.txt, for C and C++ callers) produces the same
library as the Python build script: it configures and builds on the CPU, and
libfp8kv.so exports exactly the entry points include/fp8kv.h declares."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8kv.h")


def _declared():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def _exports(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", lib], check=True,
                         capture_output=True, text=True).stdout
    names = {line.split()[-1] for line in out.splitlines() if line.strip()}
    # hipcc and clang both export one compilation-unit id per HIP source
    return sorted(n for n in names if not n.startswith("__hip_cuid_"))


@pytest.mark.skipif(shutil.which("cmake") is None or shutil.which("ninja") is None
                    or not os.path.exists("/opt/rocm/llvm/bin/clang++"),
                    reason="needs cmake, ninja and ROCm's clang")
def test_cmake_builds_the_library(tmp_path):
    build = tmp_path / "cmake"
    r = subprocess.run(["cmake", "-S", ROOT, "-B", str(build), "-G", "Ninja"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run(["cmake", "--build", str(build), "-j", "8"],
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout + r.stderr
    lib = build / "libfp8kv.so"
    assert lib.exists() and (build / "liboracle.so").exists()
    assert (build / "c_abi_driver").exists()
    assert _exports(str(lib)) == _declared()
    # the same sources get the same device flags as the Python build
    cmds = subprocess.run(["ninja", "-C", str(build), "-t", "commands", "fp8kv"],
                          capture_output=True, text=True, check=True).stdout
    hip = [c for c in cmds.splitlines() if ".hip" in c and " -c " in c]
    assert len(hip) == 8
    for c in hip:
        assert "--offload-arch=gfx950" in c and "-packed-fp32-ops" in c
        assert "-O3" in c and "-std=c++17" in c
        src = c.split(" -c ")[1]
        packed = "qk_norm_rope_packed" in src or "packed_unfused" in src
        assert ("-amdgpu-kernarg-preload-count=16" in c) == packed
