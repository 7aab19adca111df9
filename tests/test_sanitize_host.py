"""CPU sanitizer runs of the host code.

* The oracle (oracle/kvc_oracle.c) built with AddressSanitizer and
  UndefinedBehaviorSanitizer (gcc, errors fatal) runs every pin of
  tests/oracle_pins.py in a child process; a deliberately out-of-bounds
  length handed to it must end that child with an AddressSanitizer report,
  which shows the instrumentation is live.
* libkvc.so with its host code built with the same sanitizers (hipcc,
  host side only; the gfx950 device code is compiled as usual) runs the
  ABI and binding validation tests (tests/test_abi.py,
  tests/test_binding_host.py), which drive every entry point's argument
  checks and the planning arithmetic without a GPU.

Each child preloads the sanitizer runtime that its library was built
against (gcc's for the oracle, clang's for hipcc's build)."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

pytestmark = pytest.mark.slow

SAN_OPTS = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
            "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _gcc_runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


def _child(code: str, env_extra: dict, timeout: int = 600):
    env = dict(os.environ, **SAN_OPTS, **env_extra)
    env["PYTHONPATH"] = os.pathsep.join([ROOT, os.path.join(ROOT, "tests"), env.get("PYTHONPATH", "")])
    return subprocess.run([sys.executable, "-c", code], cwd=os.path.join(ROOT, "tests"), env=env,
                          capture_output=True, text=True, timeout=timeout)


@pytest.fixture(scope="module")
def sanitized_oracle(tmp_path_factory):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not shutil.which("gcc") or not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    from oracle import build as obuild
    out = str(tmp_path_factory.mktemp("san") / "libkvc_oracle_san.so")
    obuild.build(out=out, extra=["-O1", "-g", "-fno-omit-frame-pointer",
                                 "-fsanitize=address,undefined", "-fno-sanitize-recover=all"])
    return {"KVC_ORACLE_LIB": out, "LD_PRELOAD": f"{asan}:{ubsan}"}


def test_oracle_pins_under_asan_ubsan(sanitized_oracle):
    r = _child("import oracle, oracle_pins as P\n"
               f"assert oracle.LIB_PATH == {sanitized_oracle['KVC_ORACLE_LIB']!r}\n"
               "for pin in P.ALL_PINS:\n    pin()\nprint('pins ok', len(P.ALL_PINS))\n",
               sanitized_oracle)
    assert r.returncode == 0 and "pins ok" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_sanitizer_is_live_on_the_oracle(sanitized_oracle):
    """A length past the cache's end makes the oracle read beyond the array
    (a planted out-of-bounds input, on the CPU): the instrumented build must
    stop with an AddressSanitizer report."""
    r = _child("import numpy as np, oracle\n"
               "q = np.ones((1, 2, 8), np.float32)\n"
               "k = np.ones((1, 1, 4, 8), np.float32)\n"
               "oracle.decode(q, k, k.copy(), [64], 0.5, nthreads=1)\n"
               "print('no report')\n", sanitized_oracle)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stdout + r.stderr[-2000:]


def test_library_host_code_under_asan_ubsan(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc"
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not os.path.exists(hipcc) or not rt:
        pytest.skip("hipcc or clang's sanitizer runtime not installed")
    from kv_cache_gqa_amd import build as kbuild
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    out = str(tmp_path / "libkvc_san.so")
    kbuild.build(extra=["-O1", "-g", *san, "-Xarch_host", "-fno-sanitize-recover=all"],
                 out=out, objdir=str(tmp_path / "obj"), link_extra=[*san, "-shared-libsan"])
    nm = subprocess.run(["nm", "-D", out], capture_output=True, text=True).stdout
    assert "__asan_report_load" in nm and "__ubsan_handle" in nm  # the host code is instrumented
    env = dict(os.environ, **SAN_OPTS, KVC_LIB=out, LD_PRELOAD=rt[0])
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_binding_host.py"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0 and " passed" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stderr + r.stdout and "AddressSanitizer" not in r.stderr
