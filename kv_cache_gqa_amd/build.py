"""Build libkvc.so (HIP kernels + C ABI) for gfx950, in-tree.

``python -m kv_cache_gqa_amd.build`` or ``build()``.  Every HIP source is
compiled with hipcc for gfx950 only, with packed-fp32 code generation turned
off (``-Xclang -target-feature -Xclang -packed-fp32-ops``), then linked into
``kv_cache_gqa_amd/libkvc.so``.  No GPU is needed to build.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvc.so")
OBJDIR = os.path.join(PKG, "_build")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkvc)")


COMPILE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Flags of single sources.  The multi-row kernel tests for no NaN anywhere
# (masked scores are selected away before any arithmetic), so its max
# reductions need no quieting of their inputs.
FILE_FLAGS = {"prefill.hip": ["-fno-honor-nans"]}


def _compile(src: str, extra: list[str], verbose: bool, objdir: str = OBJDIR) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMPILE_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src,
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, extra: list[str] | None = None, jobs: int = 8,
          out: str = LIB, objdir: str = OBJDIR, link_extra: list[str] | None = None) -> str:
    """Compile every source and link ``out``.  ``extra`` goes to every
    compile, ``link_extra`` to the link (a sanitizer build of the host code
    passes its flags there; the default is the product library)."""
    os.makedirs(objdir, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(sources))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra or [], verbose, objdir), sources))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *(link_extra or []),
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
