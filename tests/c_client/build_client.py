"""Compiles the plain-C client of include/kvstore.h (kvstore_client.c, beside
this file) with gcc as strict C11, linked against libkvstore.so and the
oracle's liboracle.so (both must be built first).  The binary finds both
libraries through an rpath relative to itself, so the tree can move."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BINARY = os.path.join(HERE, "kvstore_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str = BINARY) -> list:
    rpath = ":".join(["$ORIGIN/../../fp8_kv_quantization_amd", "$ORIGIN/../../oracle",
                      os.path.join(ROCM, "lib")])
    return ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-pedantic",
            "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
            "-isystem", os.path.join(ROCM, "include"), os.path.join(HERE, "kvstore_client.c"),
            "-L", os.path.join(ROOT, "fp8_kv_quantization_amd"), "-lkvstore",
            "-L", os.path.join(ROOT, "oracle"), "-loracle",
            "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + rpath, "-o", out]


def build(out: str = BINARY) -> str:
    tmp = out + ".tmp"
    subprocess.run(command(tmp), check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
