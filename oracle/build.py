"""Compile the C fp64 oracle (test infrastructure) into oracle/libkvc_oracle.so.

Run as ``python oracle/build.py`` or call :func:`build`.  Plain gcc, -O2,
OpenMP over (sequence, query head) rows; no GPU code is involved.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvc_oracle.c")
LIB = os.path.join(HERE, "libkvc_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
