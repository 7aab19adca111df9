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


def build(verbose: bool = False, out: str = LIB, extra: list | None = None) -> str:
    """Compile kvc_oracle.c into ``out``; ``extra`` flags go to gcc (the
    sanitizer test builds a copy with AddressSanitizer and UBSan)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           *(extra or []), "-o", out + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
