"""Builds libkvstore.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "kvstore.hip")
HEADER = os.path.join(ROOT, "include", "kvstore.h")
LIB = os.path.join(PKG, "libkvstore.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # packed fp32 VALU forms are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def command(out: str = LIB, extra=()) -> list:
    return [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), SRC, "-o", out]


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    """Compile the HIP library (always; a few seconds).  Writes atomically."""
    tmp = out + ".tmp"
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out
