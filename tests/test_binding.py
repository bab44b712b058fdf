"""Host logic of the Python binding (CPU): the tensor-level calls refuse
tensors that are not on a GPU, and size_limit defaults to the cache's slot
count and may not exceed it."""
import pytest
import torch

import fp8_kv_quantization_amd as kv


def test_cpu_tensors_are_refused_before_any_call():
    k = torch.zeros((4, 8), dtype=torch.bfloat16)
    kc = torch.zeros((16, 8), dtype=torch.bfloat16)
    idx = torch.arange(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        kv.store_kv(k, k, kc, kc, idx)
    k3 = k.view(4, 1, 8)
    c8 = torch.zeros((16, 1, 8), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        kv.store_kv_fp8_paged(k3, k3, c8, c8, idx, page_size=16)
    sc = torch.zeros(16, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        kv.store_kv_fp8_paged_dynamic(k3, k3, c8, c8, idx, sc, sc, page_size=16)


def test_size_limit_defaults_to_and_is_bounded_by_the_slots():
    assert kv._size_limit(None, 1024) == 1024
    assert kv._size_limit(1000, 1024) == 1000
    assert kv._size_limit(1024, 1024) == 1024
    with pytest.raises(ValueError, match="size_limit"):
        kv._size_limit(1025, 1024)


def test_device_of_skips_absent_tensors():
    assert kv._device_of(None, None) is None
    with pytest.raises(ValueError, match="GPU"):
        kv._device_of(None, torch.zeros(1))


FOREIGN_CACHE_DTYPES = ["float8_e4m3fnuz", "float8_e5m2fnuz", "int8", "bool", "float16"]


@pytest.mark.parametrize("name", FOREIGN_CACHE_DTYPES)
def test_fp8_stores_refuse_caches_that_cannot_hold_the_codes(name):
    """uint8 and float8_e4m3fn caches take e4m3fn codes and float8_e5m2 caches
    e5m2 codes; any other dtype (the fnuz formats decode the same bytes with
    another bias and NaN) is refused with TypeError before the device check,
    so before anything could be launched."""
    dt = getattr(torch, name)
    k3 = torch.zeros((4, 1, 16), dtype=torch.bfloat16)
    c = torch.zeros((16, 1, 16), dtype=dt)
    sc = torch.zeros(16, dtype=torch.float32)
    idx = torch.arange(4, dtype=torch.int32)
    with pytest.raises(TypeError, match="cannot hold"):
        kv.store_kv_fp8_paged(k3, k3, c, c, idx, page_size=16)
    for fmt in ("e4m3fn", "e5m2"):
        with pytest.raises(TypeError, match="cannot hold"):
            kv.store_kv_fp8_paged(k3, k3, c, c, idx, page_size=16, fp8_format=fmt)
    with pytest.raises(TypeError, match="cannot hold"):
        kv.store_kv_fp8_paged_dynamic(k3, k3, c, c, idx, sc, sc, page_size=16)


def test_fp8_stores_match_format_and_cache_dtype():
    k3 = torch.zeros((4, 1, 16), dtype=torch.bfloat16)
    u8 = torch.zeros((16, 1, 16), dtype=torch.uint8)
    e4 = u8.view(torch.float8_e4m3fn)
    e5 = u8.view(torch.float8_e5m2)
    sc = torch.zeros(16, dtype=torch.float32)
    idx = torch.arange(4, dtype=torch.int32)
    # K and V caches of different dtypes
    with pytest.raises(TypeError, match="share one dtype"):
        kv.store_kv_fp8_paged(k3, k3, u8, e4, idx, page_size=16)
    with pytest.raises(TypeError, match="share one dtype"):
        kv.store_kv_fp8_paged_dynamic(k3, k3, e4, e5, idx, sc, sc, page_size=16)
    # a format the cache dtype does not name
    for c, fmt in ((u8, "e5m2"), (e4, "e5m2"), (e5, "e4m3fn")):
        with pytest.raises(TypeError, match="cannot hold"):
            kv.store_kv_fp8_paged(k3, k3, c, c, idx, page_size=16, fp8_format=fmt)
    with pytest.raises(ValueError, match="fp8_format"):
        kv.store_kv_fp8_paged(k3, k3, u8, u8, idx, page_size=16, fp8_format="e4m3fnuz")
    # the dynamic store writes e4m3fn codes only
    with pytest.raises(TypeError, match="e4m3fn"):
        kv.store_kv_fp8_paged_dynamic(k3, k3, e5, e5, idx, sc, sc, page_size=16)
    # accepted pairs get past the dtype check (then refused as CPU tensors)
    for c, fmt in ((u8, None), (e4, None), (e5, None), (u8, "e4m3fn"), (e5, "e5m2")):
        assert kv._fp8_format(c, c, fmt) == (fmt or ("e5m2" if c is e5 else "e4m3fn"))
        with pytest.raises(ValueError, match="GPU"):
            kv.store_kv_fp8_paged(k3, k3, c, c, idx, page_size=16, fp8_format=fmt)
    for c in (u8, e4):
        with pytest.raises(ValueError, match="GPU"):
            kv.store_kv_fp8_paged_dynamic(k3, k3, c, c, idx, sc, sc, page_size=16)


def test_import_without_the_library_raises(tmp_path):
    """The package has no CPU or torch fallback: a copy of it without
    libkvstore.so refuses to import."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "fp8_kv_quantization_amd"
    pkg.mkdir()
    shutil.copy(kv.__file__, pkg / "__init__.py")
    r = subprocess.run([sys.executable, "-c", "import fp8_kv_quantization_amd"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libkvstore.so is not built" in r.stderr
