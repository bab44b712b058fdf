"""Helpers for the GPU parity tests: moving kvgen inputs to the device,
calling the library through its C ABI, and comparing device caches with the
oracle's host caches in bounded chunks."""
from __future__ import annotations

import numpy as np
import torch

import fp8_kv_quantization_amd as kv

DEV = torch.device("cuda:0")
CHUNK_BYTES = 256 << 20


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def f32_dev(bits):
    if bits is None:
        return None
    return to_dev(np.array([bits], dtype=np.uint32).view(np.float32))


def sentinel_cache(rows: int, row_bytes: int) -> torch.Tensor:
    return torch.full((rows, row_bytes), 0xFF, dtype=torch.uint8, device=DEV)


def stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def idx_code(a: np.ndarray) -> int:
    return kv.IDX_I64 if a.dtype == np.int64 else kv.IDX_I32


def run_copy(case, kc, vc, idx_dev=None, size_limit=None, batch=None, idx_stride=1):
    """kvstore_copy through the C ABI for a kvgen copy case."""
    k = to_dev(case.k)
    v = to_dev(case.v)
    idx = to_dev(case.indices) if idx_dev is None else idx_dev
    st = kv.kvstore_copy(k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                         idx.data_ptr(), idx_code(case.indices), idx_stride, case.row_bytes,
                         case.in_stride_bytes, case.in_stride_bytes, kc.stride(0),
                         case.num_tokens if batch is None else batch,
                         case.slots if size_limit is None else size_limit, stream())
    return st


def run_fp8(case, kc, vc, idx_dev=None, size_limit=None, kc_strides=None, vc_strides=None,
            in_strides=None, k_dev=None, v_dev=None, batch=None, idx_stride=1, fmt="e4m3fn"):
    """kvstore_fp8_paged through the C ABI for a kvgen fp8 case (contiguous
    [slots, H*D] byte caches unless strides are given)."""
    H, D, P = case.num_heads, case.head_dim, case.page_size
    row = H * D
    k = to_dev(case.k) if k_dev is None else k_dev
    v = to_dev(case.v) if v_dev is None else v_dev
    idx = to_dev(case.indices) if idx_dev is None else idx_dev
    ks = in_strides or (case.in_stride_bytes, 2 * D)
    kcs = kc_strides or (P * row, row, D)
    vcs = vc_strides or kcs
    ik, iv = f32_dev(case.inv_k_bits), f32_dev(case.inv_v_bits)
    entry = kv.kvstore_fp8_paged_e5m2 if fmt == "e5m2" else kv.kvstore_fp8_paged
    st = entry(
        k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(), idx.data_ptr(),
        idx_code(case.indices), idx_stride, kv.SRC_FP16 if case.src_dtype == "fp16" else kv.SRC_BF16,
        H, D, ks[0], ks[1], ks[0], ks[1], kcs[0], kcs[1], kcs[2], vcs[0], vcs[1], vcs[2],
        case.num_tokens if batch is None else batch, case.slots if size_limit is None else size_limit,
        P, None if ik is None else ik.data_ptr(), None if iv is None else iv.data_ptr(), stream())
    # keep scale tensors alive until the work is done
    torch.cuda.current_stream().synchronize()
    return st


def assert_cache_equal(dev: torch.Tensor, host: np.ndarray, what: str = "cache"):
    """Byte-compare a device cache with a host array, in bounded chunks."""
    flat_d = dev.reshape(-1)
    flat_h = host.reshape(-1)
    assert flat_d.numel() == flat_h.size, (flat_d.numel(), flat_h.size)
    n = flat_h.size
    for s in range(0, n, CHUNK_BYTES):
        e = min(n, s + CHUNK_BYTES)
        got = flat_d[s:e].cpu().numpy()
        want = flat_h[s:e]
        if not np.array_equal(got, want):
            bad = np.nonzero(got != want)[0]
            first = int(bad[0]) + s
            raise AssertionError(
                f"{what}: {bad.size} bytes differ in [{s}, {e}); first at byte {first}: "
                f"got 0x{int(got[bad[0]]):02x} want 0x{int(want[bad[0]]):02x}")


def check_flag():
    """(status, first_bad, count) from kvstore_check_error on the current stream."""
    return kv.kvstore_check_error(stream())
