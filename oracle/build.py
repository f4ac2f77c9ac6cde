"""Compile the C oracle into ``oracle/liblowbit_oracle.so`` with gcc.

Test infrastructure: building the checker is not using it.  Flags keep every
float operation a single correctly rounded IEEE operation (no contraction into
FMA, no fast-math, SSE arithmetic on x86-64).
"""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "liblowbit_oracle.so")


def build() -> str:
    src = os.path.join(_HERE, "lowbit_oracle.c")
    out = library_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
