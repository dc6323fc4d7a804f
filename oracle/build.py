"""Builds the CPU oracle library (plain gcc, no fast-math) next to its source.

Test infrastructure: the oracle is only ever called by the tests, the smoke
check and the benchmark's CPU-baseline leg.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(HERE, "liboracle.so")


def build() -> str:
    src = os.path.join(HERE, "attn_oracle.c")
    out = library_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-pthread",
           src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
