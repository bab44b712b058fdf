"""Builds libkvstore.so in-tree with hipcc for gfx950, and its CPython
binding (_kvstore_py, gcc, linked against libkvstore.so)."""
from __future__ import annotations

import os
import subprocess
import sysconfig

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "kvstore.hip")
HEADER = os.path.join(ROOT, "include", "kvstore.h")
LIB = os.path.join(PKG, "libkvstore.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
PY_SRC = os.path.join(PKG, "csrc", "kvstore_py.c")
PY_EXT = os.path.join(PKG, "_kvstore_py" + sysconfig.get_config_var("EXT_SUFFIX"))

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # packed fp32 VALU forms are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def command(out: str = LIB, extra=()) -> list:
    return [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), SRC, "-o", out]


def binding_command(out: str = PY_EXT) -> list:
    return ["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-Wall", "-Wextra",
            "-D__HIP_PLATFORM_AMD__", "-I", sysconfig.get_paths()["include"],
            "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"),
            PY_SRC, "-L", PKG, "-lkvstore", "-Wl,-rpath,$ORIGIN", "-o", out]


def _run(cmd, out, what, verbose):
    tmp = out + ".tmp"
    cmd = [tmp if c == out else c for c in cmd]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{what} failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    """Compile the HIP library and, for the in-tree library, the CPython
    binding (always; a few seconds).  Writes atomically."""
    _run(command(out, extra), out, "hipcc", verbose)
    if out == LIB:
        _run(binding_command(), PY_EXT, "gcc (binding)", verbose)
    return out
