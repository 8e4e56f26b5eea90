"""Build ``tests/c_abi_driver`` (a plain C caller of libfp8kv.so, test
infrastructure) with the host C compiler against the HIP runtime.

    python -m tests.build_c_driver
"""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_driver.c")
OUT = os.path.join(HERE, "c_abi_driver")


def build() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no host C compiler")
    pkg = os.path.join(ROOT, "fp8_kv_cache_slot_amd")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Werror",
           # the HIP runtime headers need the platform named when a plain C
           # compiler includes them
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
           "-I", os.path.join(ROOT, "include"), SRC, "-o", OUT,
           "-L", pkg, "-lfp8kv", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../fp8_kv_cache_slot_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the C driver failed:\n{r.stderr}")
    return OUT


if __name__ == "__main__":
    print(build())
