import importlib.util
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads")


def pytest_sessionstart(session):
    # Build the HIP library and its binding only when they are not built (a
    # fresh checkout): tests load what is built and never rebuild them.
    lib = os.path.join(ROOT, "fp8_kv_quantization_amd", "libkvstore.so")
    pkg = os.path.join(ROOT, "fp8_kv_quantization_amd")
    has_binding = any(f.startswith("_kvstore_py") and f.endswith(".so") for f in os.listdir(pkg))
    if not os.path.exists(lib) or not has_binding:
        path = os.path.join(ROOT, "fp8_kv_quantization_amd", "_build.py")
        spec = importlib.util.spec_from_file_location("_kvstore_build", path)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    # The plain-C client of the ABI, likewise only when missing.
    client = os.path.join(ROOT, "tests", "c_client", "kvstore_client")
    if not os.path.exists(client):
        import oracle
        oracle.build()
        path = os.path.join(ROOT, "tests", "c_client", "build_client.py")
        spec = importlib.util.spec_from_file_location("_kvstore_client_build", path)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


def _gpu_present() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_present():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
