"""Build the oracle's C library with gcc (test infrastructure only).

Plain -O2 for the baseline x86-64 instruction set, so the library built in one
container also runs on another host's CPU.  OpenMP parallelises over rows.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lora_oracle.c")
LIB = os.path.join(HERE, "liblora_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-Wextra",
           SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
