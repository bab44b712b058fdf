"""CPU oracle for the KV-cache store (ctypes wrapper over kvstore_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check and
by the benchmark's CPU-baseline leg, never by the product path.  It shares no
code with the HIP library; both are fed the same seeded inputs and their
outputs are compared byte for byte.

The C source states what each function follows on the pages (sglang
"kvcache.cuh" store_kvcache for the copy, sglang "trtllm_fp8_kv_kernel.py"
_fused_fp8_set_kv_buffer_kernel for the fused FP8 paged store) and the
reading taken for the e4m3fn cast (round to nearest even, saturate to +-448).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "kvstore_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")
BUILD_CMD = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-shared",
             "-fPIC", SRC, "-o", LIB, "-lm"]

_lib = None


def build(force: bool = False) -> str:
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        subprocess.run(BUILD_CMD, check=True)
    return LIB


def load(path: Optional[str] = None):
    """Load the oracle library (building it with gcc if it is not there)."""
    global _lib
    if path is not None:
        return _bind(C.CDLL(path))
    if _lib is None:
        build()
        _lib = _bind(C.CDLL(LIB))
    return _lib


def _bind(lib):
    vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int
    lib.oracle_e4m3fn_from_float.argtypes = [C.c_float]
    lib.oracle_e4m3fn_from_float.restype = C.c_uint8
    lib.oracle_src_to_float.argtypes = [C.c_uint16, i32]
    lib.oracle_src_to_float.restype = C.c_float
    lib.oracle_mul_f32.argtypes = [C.c_float, C.c_float]
    lib.oracle_mul_f32.restype = C.c_float
    lib.oracle_quantize.argtypes = [vp, i64, i32, vp, vp]
    lib.oracle_quantize.restype = None
    lib.oracle_e4m3fn_array.argtypes = [vp, i64, vp]
    lib.oracle_e4m3fn_array.restype = None
    lib.oracle_copy.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, i64, i64, i64, i64,
                                vp, vp]
    lib.oracle_copy.restype = i64
    lib.oracle_fp8_paged.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i64, i64,
                                     i64, i64, i64, i64, i64, i64, i64, i64, i64, i64,
                                     i64, i64, i64, vp, vp, vp, vp]
    lib.oracle_fp8_paged.restype = i64
    lib.oracle_e5m2_from_float.argtypes = [C.c_float]
    lib.oracle_e5m2_from_float.restype = C.c_uint8
    lib.oracle_e5m2_array.argtypes = [vp, i64, vp]
    lib.oracle_e5m2_array.restype = None
    lib.oracle_quantize_e5m2.argtypes = [vp, i64, i32, vp, vp]
    lib.oracle_quantize_e5m2.restype = None
    lib.oracle_fp8_paged_e5m2.argtypes = lib.oracle_fp8_paged.argtypes
    lib.oracle_fp8_paged_e5m2.restype = i64
    lib.oracle_fp8_paged_dynamic.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i64, i64,
                                             i64, i64, i64, i64, i64, i64, i64, i64, i64, i64,
                                             vp, vp, i64, i64, i64, i64, i64, i64, i32,
                                             i64, i64, i64, vp, vp]
    lib.oracle_fp8_paged_dynamic.restype = i64
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _f32_box(bits: Optional[int]):
    if bits is None:
        return None
    return np.array([bits], dtype=np.uint32).view(np.float32)


# --------------------------------------------------------------------------
# Element helpers
# --------------------------------------------------------------------------

def e4m3fn(y: np.ndarray, lib=None) -> np.ndarray:
    """Saturating round-to-nearest-even e4m3fn codes of fp32 values."""
    lib = lib or load()
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib.oracle_e4m3fn_array(_ptr(y), y.size, _ptr(out))
    return out


def e5m2(y: np.ndarray, lib=None) -> np.ndarray:
    """Saturating round-to-nearest-even e5m2 codes of fp32 values."""
    lib = lib or load()
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib.oracle_e5m2_array(_ptr(y), y.size, _ptr(out))
    return out


def quantize(bits: np.ndarray, src_dtype: str, inv_bits: Optional[int], lib=None,
             fmt: str = "e4m3fn") -> np.ndarray:
    """fmt(decode(bits) * inv) for each 16-bit input pattern (fmt e4m3fn or e5m2)."""
    lib = lib or load()
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.uint8)
    inv = _f32_box(inv_bits)
    fn = lib.oracle_quantize_e5m2 if fmt == "e5m2" else lib.oracle_quantize
    fn(_ptr(bits), bits.size, int(src_dtype == "fp16"), None if inv is None else _ptr(inv),
       _ptr(out))
    return out


def src_to_float(bits: np.ndarray, src_dtype: str, lib=None) -> np.ndarray:
    lib = lib or load()
    f = lib.oracle_src_to_float
    flag = int(src_dtype == "fp16")
    return np.array([f(int(b), flag) for b in np.asarray(bits).ravel()],
                    dtype=np.float32).reshape(np.shape(bits))


# --------------------------------------------------------------------------
# Stores (numpy arrays in, caches mutated in place)
# --------------------------------------------------------------------------

def copy(k: np.ndarray, v: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
         indices: np.ndarray, *, row_bytes: int, k_stride: int, v_stride: int,
         cache_stride: int, size_limit: int, batch: Optional[int] = None,
         idx_stride: int = 1, lib=None):
    """Scatter copy into byte caches.  Strides are bytes, idx_stride elements.
    Returns (rows_written, first_bad_token, bad_count)."""
    lib = lib or load()
    fb = np.zeros(1, dtype=np.int64)
    bc = np.zeros(1, dtype=np.uint64)
    is64 = int(indices.dtype == np.int64)
    if batch is None:
        batch = (indices.size + idx_stride - 1) // idx_stride
    n = lib.oracle_copy(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(indices), is64,
                        idx_stride, row_bytes, k_stride, v_stride, cache_stride, batch,
                        size_limit, _ptr(fb), _ptr(bc))
    return int(n), int(fb[0]), int(bc[0])


def fp8_paged(k: np.ndarray, v: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
              indices: np.ndarray, *, src_dtype: str, num_heads: int, head_dim: int,
              k_strides, v_strides, kc_strides, vc_strides, size_limit: int, page_size: int,
              inv_k_bits: Optional[int], inv_v_bits: Optional[int],
              batch: Optional[int] = None, idx_stride: int = 1, lib=None, fmt: str = "e4m3fn"):
    """Fused FP8 paged store (e4m3fn or e5m2 caches).  k_strides/v_strides =
    (token, head) in bytes; kc_strides/vc_strides = (page, offset, head) in
    bytes.  Returns (rows_written, first_bad_token, bad_count)."""
    lib = lib or load()
    fb = np.zeros(1, dtype=np.int64)
    bc = np.zeros(1, dtype=np.uint64)
    ik = _f32_box(inv_k_bits)
    iv = _f32_box(inv_v_bits)
    is64 = int(indices.dtype == np.int64)
    if batch is None:
        batch = (indices.size + idx_stride - 1) // idx_stride
    fn = lib.oracle_fp8_paged_e5m2 if fmt == "e5m2" else lib.oracle_fp8_paged
    n = fn(
        _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(indices), is64, idx_stride,
        int(src_dtype == "fp16"), num_heads, head_dim, k_strides[0], k_strides[1],
        v_strides[0], v_strides[1], kc_strides[0], kc_strides[1], kc_strides[2],
        vc_strides[0], vc_strides[1], vc_strides[2], batch, size_limit, page_size,
        None if ik is None else _ptr(ik), None if iv is None else _ptr(iv), _ptr(fb), _ptr(bc))
    return int(n), int(fb[0]), int(bc[0])


def fp8_paged_dynamic(k, v, k_cache, v_cache, indices, k_scales, v_scales, *, src_dtype,
                      num_heads, head_dim, k_strides, v_strides, kc_strides, vc_strides,
                      ks_strides, vs_strides, per_head, size_limit, page_size,
                      batch=None, idx_stride=1, lib=None):
    """Fused FP8 paged store with dynamic scales.  ks_strides/vs_strides =
    (page, offset, head) byte strides of the fp32 scale caches (k_scales /
    v_scales are any host arrays, written as raw bytes).
    Returns (rows_written, first_bad_token, bad_count)."""
    lib = lib or load()
    fb = np.zeros(1, dtype=np.int64)
    bc = np.zeros(1, dtype=np.uint64)
    is64 = int(indices.dtype == np.int64)
    if batch is None:
        batch = (indices.size + idx_stride - 1) // idx_stride
    n = lib.oracle_fp8_paged_dynamic(
        _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(indices), is64, idx_stride,
        int(src_dtype == "fp16"), num_heads, head_dim, k_strides[0], k_strides[1],
        v_strides[0], v_strides[1], kc_strides[0], kc_strides[1], kc_strides[2],
        vc_strides[0], vc_strides[1], vc_strides[2], _ptr(k_scales), _ptr(v_scales),
        ks_strides[0], ks_strides[1], ks_strides[2], vs_strides[0], vs_strides[1],
        vs_strides[2], int(bool(per_head)), batch, size_limit, page_size, _ptr(fb), _ptr(bc))
    return int(n), int(fb[0]), int(bc[0])


def run_case_dynamic(case, per_head: bool, lib=None):
    """Dynamic-scale store of a kvgen fp8 case into contiguous sentinel caches
    ([slots, H*D] bytes) and contiguous scale caches ([slots, groups] fp32,
    filled with the 0xFFFFFFFF pattern).  Returns (k_cache, v_cache, k_scales,
    v_scales, status)."""
    row = case.cache_row_bytes
    H, D, P = case.num_heads, case.head_dim, case.page_size
    G = H if per_head else 1
    kc = np.full((case.slots, row), 0xFF, dtype=np.uint8)
    vc = np.full_like(kc, 0xFF)
    ks = np.full((case.slots, G), 0xFFFFFFFF, dtype=np.uint32)
    vs = np.full_like(ks, 0xFFFFFFFF)
    cs = (P * row, row, D)
    ss = (P * G * 4, G * 4, 4)
    st = fp8_paged_dynamic(case.k, case.v, kc, vc, case.indices, ks, vs,
                           src_dtype=case.src_dtype, num_heads=H, head_dim=D,
                           k_strides=(case.in_stride_bytes, 2 * D),
                           v_strides=(case.in_stride_bytes, 2 * D), kc_strides=cs,
                           vc_strides=cs, ks_strides=ss, vs_strides=ss, per_head=per_head,
                           size_limit=case.slots, page_size=P, lib=lib)
    return kc, vc, ks, vs, st


# --------------------------------------------------------------------------
# Whole-workload conveniences (kvgen.Case in, host caches out)
# --------------------------------------------------------------------------

def run_case(case, k_cache: Optional[np.ndarray] = None, v_cache: Optional[np.ndarray] = None,
             indices: Optional[np.ndarray] = None, lib=None, fmt: str = "e4m3fn"):
    """Run the oracle on a kvgen.Case with contiguous sentinel-filled caches
    (``[slots, cache_row_bytes]`` uint8) unless caches are given.
    Returns (k_cache, v_cache, (rows_written, first_bad, bad_count))."""
    row = case.cache_row_bytes
    if k_cache is None:
        k_cache = np.full((case.slots, row), 0xFF, dtype=np.uint8)
    if v_cache is None:
        v_cache = np.full((case.slots, row), 0xFF, dtype=np.uint8)
    idx = case.indices if indices is None else indices
    if case.kind == "copy":
        st = copy(case.k, case.v, k_cache, v_cache, idx, row_bytes=case.row_bytes,
                  k_stride=case.in_stride_bytes, v_stride=case.in_stride_bytes,
                  cache_stride=row, size_limit=case.slots, lib=lib)
    else:
        H, D, P = case.num_heads, case.head_dim, case.page_size
        cs = (P * row, row, D)
        st = fp8_paged(case.k, case.v, k_cache, v_cache, idx, src_dtype=case.src_dtype,
                       num_heads=H, head_dim=D, k_strides=(case.in_stride_bytes, 2 * D),
                       v_strides=(case.in_stride_bytes, 2 * D), kc_strides=cs, vc_strides=cs,
                       size_limit=case.slots, page_size=P, inv_k_bits=case.inv_k_bits,
                       inv_v_bits=case.inv_v_bits, lib=lib, fmt=fmt)
    return k_cache, v_cache, st
