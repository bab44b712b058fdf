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
