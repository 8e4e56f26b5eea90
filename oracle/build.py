"""Build the CPU oracle (test infrastructure): ``oracle.cpp`` -> ``liboracle.so``.

Plain g++, no fast-math, so that double arithmetic and round-to-nearest-even
are exactly what the source says.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build() -> str:
    out = os.path.join(HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["g++", "-std=c++17", "-O2", "-fno-fast-math", "-ffp-contract=off",
           "-fPIC", "-shared", "-Wall", "-Wextra",
           os.path.join(HERE, "oracle.cpp"), "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
