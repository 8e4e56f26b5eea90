"""Build the CPU oracle (test infrastructure): ``oracle.cpp`` -> ``liboracle.so``.

Plain g++, no fast-math, so that double arithmetic and round-to-nearest-even
are exactly what the source says.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(src: str | None = None, out: str | None = None) -> str:
    """Compile ``src`` (default: oracle.cpp here) to the shared library
    ``out`` (default: liboracle.so here).  The header is taken from this
    directory either way."""
    src = src or os.path.join(HERE, "oracle.cpp")
    out = out or os.path.join(HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["g++", "-std=c++17", "-O2", "-fno-fast-math", "-ffp-contract=off",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-I", HERE, src, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
