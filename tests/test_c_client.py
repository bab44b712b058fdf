"""The C ABI from plain C, with no Python between the caller and the library.

include/kvstore.h compiles as strict C99 and C11 on its own, and the C
program tests/c_client/kvstore_client.c, linked against libkvstore.so, gets
the documented status for every argument rule of every entry point (CPU: each
of those calls returns before any launch) and, on the GPU, stores through
every entry point into hipMalloc'd buffers that match the oracle byte for
byte, error flag included.
"""
import importlib.util
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _builder():
    path = os.path.join(HERE, "c_client", "build_client.py")
    spec = importlib.util.spec_from_file_location("_kvstore_client_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _client() -> str:
    b = _builder()
    if not os.path.exists(b.BINARY):
        b.build()
    return b.BINARY


@pytest.mark.parametrize("std", ["c99", "c11"])
def test_header_compiles_alone_as_strict_c(tmp_path, std):
    tu = tmp_path / "tu.c"
    tu.write_text('#include "kvstore.h"\n'
                  "int main(void) { return kvstore_strerror(KVSTORE_OK) == 0; }\n")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    r = subprocess.run(["gcc", f"-std={std}", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-D__HIP_PLATFORM_AMD__", "-fsyntax-only", "-I",
                        os.path.join(ROOT, "include"), "-isystem", os.path.join(rocm, "include"),
                        str(tu)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr


def test_c_client_argument_checks():
    r = subprocess.run([_client(), "validate"], capture_output=True, text=True, timeout=60)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "validate: 0 failure(s)" in r.stdout


@pytest.mark.gpu
def test_c_client_stores_match_oracle():
    print("[gpu-case] C client, every entry point", flush=True)
    r = subprocess.run([_client(), "gpu"], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "gpu: 0 failure(s)" in r.stdout
