"""Python binding of libkvstore, the MI355X (gfx950) KV-cache store.

Argument marshalling only: every step of a store runs in the HIP kernels of
``libkvstore.so`` (built from ``csrc/kvstore.hip``); the functions named like
the C ABI come from the CPython extension ``_kvstore_py`` (``csrc/kvstore_py.c``),
which converts Python ints and calls the library.  There is no fallback: if
either is not built, importing this package raises.

Low level (same names and arguments as the C ABI in ``include/kvstore.h``;
pointers are ints, strides in bytes unless stated):

    kvstore_copy(...)        -> status
    kvstore_fp8_paged(...)   -> status
    kvstore_fp8_paged_e5m2(...) -> status
    kvstore_fp8_paged_dynamic(...) -> status
    kvstore_check_error(stream) -> (status, first_bad_token, bad_count)
    kvstore_take_error(out_ptr, stream) -> status   (graph-capturable, no sync)
    kvstore_strerror(status) -> str

Tensor level (torch tensors on the GPU; the current stream is used):

    store_kv(k, v, k_cache, v_cache, indices, size_limit=None)
        sglang "kvcache.cuh" store_kvcache: k/v [T, D] (dim stride 1),
        caches [S, D] with a shared row stride, indices [T] int32/int64.
    store_kv_fp8_paged(k, v, k_cache, v_cache, cache_loc, page_size=16,
                       inv_k_scale=None, inv_v_scale=None, size_limit=None)
        sglang "trtllm_fp8_kv_kernel.py" fused_fp8_set_kv_buffer: k/v
        [T, H, D] or [T, H*D] bf16/fp16; caches uint8 (e4m3fn bytes) or
        float8_e4m3fn, flat [slots, H, D] or paged [pages, page_size, H, D];
        inverse scales as fp32 device tensors (one element) or None.  uint8
        and float8_e4m3fn caches get e4m3fn codes, float8_e5m2 caches e5m2
        codes; any other cache dtype (the fnuz formats among them) raises
        TypeError, as do K and V caches of different dtypes.
    store_kv_fp8_paged_dynamic(k, v, k_cache, v_cache, cache_loc,
                               k_scale_cache, v_scale_cache, per_head=False,
                               page_size=16, size_limit=None)
        the same store with scales computed per token (or per token and head)
        and written as fp32 into scale caches shaped [slots] / [slots, H]
        (flat) or [pages, page_size] / [pages, page_size, H] (paged); the
        caches hold e4m3fn codes (uint8 or float8_e4m3fn).
"""
from __future__ import annotations

import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvstore.so")

OK = 0
ERR_NULL = -1
ERR_SHAPE = -2
ERR_ALIGN = -3
ERR_DTYPE = -4
ERR_HIP = -5
ERR_OOB = -6
IDX_I32 = 0
IDX_I64 = 1
SRC_BF16 = 0
SRC_FP16 = 1
SCALE_PER_TOKEN = 0
SCALE_PER_TOKEN_HEAD = 1

EXPORTED = ("kvstore_copy", "kvstore_fp8_paged", "kvstore_fp8_paged_e5m2",
            "kvstore_fp8_paged_dynamic", "kvstore_check_error", "kvstore_take_error",
            "kvstore_strerror")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")

# ---------------------------------------------------------------------------
# C ABI, one to one: the same names and arguments as include/kvstore.h
# (pointers as ints, None for NULL; strides in bytes unless stated; the
# trailing stream is optional).  Each returns the C status; the error check
# returns (status, first_bad_token, bad_count).
# ---------------------------------------------------------------------------
from ._kvstore_py import (kvstore_check_error, kvstore_copy,  # noqa: E402,F401
                          kvstore_fp8_paged, kvstore_fp8_paged_dynamic,
                          kvstore_fp8_paged_e5m2, kvstore_strerror, kvstore_take_error)


class KVStoreError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {kvstore_strerror(status)} (status {status})" if what
                         else f"{kvstore_strerror(status)} (status {status})")


# ---------------------------------------------------------------------------
# Tensor level
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_handle(stream, device=None):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def _idx_code(indices) -> int:
    torch = _torch()
    if indices.dtype == torch.int32:
        return IDX_I32
    if indices.dtype == torch.int64:
        return IDX_I64
    raise TypeError(f"indices must be int32 or int64, got {indices.dtype}")


def _device_of(*tensors):
    """The one GPU that holds every tensor (the store runs there)."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("every tensor must be a GPU tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"all tensors must be on one GPU (found {dev} and {t.device})")
    return dev


def _size_limit(size_limit, slots):
    """size_limit, defaulting to the cache's slot count and never beyond it
    (the kernels bound indices by it, so a larger value could write past the
    cache tensor)."""
    limit = slots if size_limit is None else int(size_limit)
    if limit > slots:
        raise ValueError(f"size_limit ({limit}) exceeds the cache's {slots} slots")
    return limit


def store_kv(k, v, k_cache, v_cache, indices, size_limit=None, stream=None) -> None:
    """Scatter copy: k_cache[indices[t]] = k[t], v_cache[indices[t]] = v[t]."""
    torch = _torch()
    dev = _device_of(k, v, k_cache, v_cache, indices)
    if k.dim() != 2 or v.dim() != 2 or k_cache.dim() != 2 or v_cache.dim() != 2:
        raise ValueError("k, v, k_cache, v_cache must be 2-D")
    if indices.dim() != 1 or indices.shape[0] != k.shape[0] or v.shape[0] != k.shape[0]:
        raise ValueError("indices must be [T] with T = k.shape[0] = v.shape[0]")
    if not (k.dtype == v.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("k, v and the caches must share one dtype")
    D = k.shape[1]
    if v.shape[1] != D or k_cache.shape[1] != D or v_cache.shape[1] != D:
        raise ValueError("row width mismatch")
    if any(t.stride(1) != 1 for t in (k, v, k_cache, v_cache)):
        raise ValueError("rows must be contiguous (dim stride 1)")
    if k_cache.stride(0) != v_cache.stride(0):
        raise ValueError("k_cache and v_cache must share one row stride")
    if k_cache.shape[0] != v_cache.shape[0]:
        raise ValueError("k_cache and v_cache must have the same number of slots")
    es = k.element_size()
    limit = _size_limit(size_limit, k_cache.shape[0])
    with torch.cuda.device(dev):
        st = kvstore_copy(k.data_ptr(), v.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                          indices.data_ptr(), _idx_code(indices),
                          indices.stride(0) if k.shape[0] else 1, D * es, k.stride(0) * es,
                          v.stride(0) * es, k_cache.stride(0) * es, k.shape[0], limit,
                          _stream_handle(stream, dev))
    if st != OK:
        raise KVStoreError(st, "kvstore_copy")


def _fp8_format(k_cache, v_cache, fp8_format=None, allowed=("e4m3fn", "e5m2")):
    """The FP8 code format the two caches receive.  Both caches must share
    one dtype.  e4m3fn codes go into uint8 or float8_e4m3fn caches, e5m2
    codes into float8_e5m2 caches; fp8_format defaults to the one the cache
    dtype names (e4m3fn for uint8).  Anything else, the fnuz formats (another
    exponent bias and NaN encoding) included, raises TypeError."""
    torch = _torch()
    if k_cache.dtype != v_cache.dtype:
        raise TypeError(f"k_cache and v_cache must share one dtype ({k_cache.dtype} != "
                        f"{v_cache.dtype})")
    dt = k_cache.dtype
    holds = {"e4m3fn": (torch.uint8, torch.float8_e4m3fn), "e5m2": (torch.float8_e5m2,)}
    if fp8_format is None:
        fp8_format = "e5m2" if dt == torch.float8_e5m2 else "e4m3fn"
    if fp8_format not in holds:
        raise ValueError(f"unknown fp8_format {fp8_format!r}")
    if fp8_format not in allowed:
        raise TypeError(f"this store writes {' or '.join(allowed)} codes, not {fp8_format}")
    if dt not in holds[fp8_format]:
        raise TypeError(f"a {dt} cache cannot hold {fp8_format} codes: e4m3fn codes go into "
                        "uint8 or float8_e4m3fn caches, e5m2 codes into float8_e5m2 caches")
    return fp8_format


def _cache_strides(cache, page_size):
    """(num_heads, head_dim, slots, (page, offset, head) byte strides) of a
    flat [slots, H, D] or paged [pages, page_size, H, D] byte cache."""
    if cache.element_size() != 1:
        raise TypeError("FP8 caches must be 1-byte elements (uint8 or float8_e4m3fn)")
    if cache.dim() == 3:
        slots, H, D = cache.shape
        if slots % page_size:
            raise ValueError(f"a flat cache of {slots} slots does not split into pages of {page_size}")
        if cache.stride(2) != 1:
            raise ValueError("cache dim stride must be 1")
        return H, D, slots, (cache.stride(0) * page_size, cache.stride(0), cache.stride(1))
    if cache.dim() == 4:
        pages, ps, H, D = cache.shape
        if ps != page_size:
            raise ValueError(f"the paged cache holds {ps} slots per page, not page_size={page_size}")
        if cache.stride(3) != 1:
            raise ValueError("cache dim stride must be 1")
        return H, D, pages * ps, (cache.stride(0), cache.stride(1), cache.stride(2))
    raise ValueError(f"a cache is 3-D (flat) or 4-D (paged), not {cache.dim()}-D")


def _input_strides(x, H, D):
    """(token, head) byte strides of [T, H, D] or [T, H*D] input."""
    es = x.element_size()
    if x.dim() == 3:
        if x.shape[1] != H or x.shape[2] != D:
            raise ValueError(f"input shape {tuple(x.shape)} does not match cache heads/dim {H}x{D}")
        if x.stride(2) != 1:
            raise ValueError("input dim stride must be 1")
        return x.stride(0) * es, x.stride(1) * es
    if x.dim() == 2:
        if x.shape[1] != H * D:
            raise ValueError(f"input width {x.shape[1]} != {H * D}")
        if x.stride(1) != 1:
            raise ValueError("input dim stride must be 1")
        return x.stride(0) * es, D * es
    raise ValueError(f"k and v are 2-D [T, H*D] or 3-D [T, H, D], not {x.dim()}-D")


def store_kv_fp8_paged(k, v, k_cache, v_cache, cache_loc, page_size=16, inv_k_scale=None,
                       inv_v_scale=None, size_limit=None, stream=None, fp8_format=None) -> None:
    """Fused FP8 quantise + paged store (scales are fp32 *inverse* scales on
    the device; None means unscaled).  fp8_format "e4m3fn" or "e5m2"; by
    default e5m2 for float8_e5m2 caches, else e4m3fn."""
    torch = _torch()
    fp8_format = _fp8_format(k_cache, v_cache, fp8_format)
    entry = kvstore_fp8_paged_e5m2 if fp8_format == "e5m2" else kvstore_fp8_paged
    dev = _device_of(k, v, k_cache, v_cache, cache_loc, inv_k_scale, inv_v_scale)
    if k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16:
        src = SRC_BF16
    elif k.dtype == torch.float16 and v.dtype == torch.float16:
        src = SRC_FP16
    else:
        raise TypeError("k and v must both be bfloat16 or both float16")
    H, D, slots, kcs = _cache_strides(k_cache, page_size)
    H2, D2, slots2, vcs = _cache_strides(v_cache, page_size)
    if (H, D, slots) != (H2, D2, slots2):
        raise ValueError("k_cache and v_cache shapes differ")
    ks = _input_strides(k, H, D)
    vs = _input_strides(v, H, D)
    T = k.shape[0]
    if v.shape[0] != T or cache_loc.dim() != 1 or cache_loc.shape[0] != T:
        raise ValueError("cache_loc must be [T] with T = k.shape[0] = v.shape[0]")
    ptrs = []
    for s in (inv_k_scale, inv_v_scale):
        if s is None:
            ptrs.append(None)
            continue
        if s.dtype != torch.float32 or s.numel() != 1 or not s.is_cuda:
            raise TypeError("inverse scales must be one-element fp32 GPU tensors")
        ptrs.append(s.data_ptr())
    limit = _size_limit(size_limit, slots)
    with torch.cuda.device(dev):
        st = entry(k.data_ptr(), v.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                   cache_loc.data_ptr(), _idx_code(cache_loc), cache_loc.stride(0) if T else 1,
                   src, H, D, ks[0], ks[1], vs[0], vs[1], kcs[0], kcs[1], kcs[2], vcs[0], vcs[1],
                   vcs[2], T, limit, page_size, ptrs[0], ptrs[1], _stream_handle(stream, dev))
    if st != OK:
        raise KVStoreError(st, entry.__name__)


def _scale_strides(sc, per_head, H, page_size):
    """(page, offset, head) byte strides of a flat [slots(, H)] or paged
    [pages, page_size(, H)] fp32 scale cache."""
    torch = _torch()
    if sc.dtype != torch.float32 or not sc.is_cuda:
        raise TypeError("scale caches must be float32 GPU tensors")
    want = 2 if per_head else 1
    if sc.dim() == want:                       # flat
        if per_head and sc.shape[1] != H:
            raise ValueError("per-head scale cache must be [slots, H]")
        return (sc.stride(0) * 4 * page_size, sc.stride(0) * 4,
                sc.stride(1) * 4 if per_head else 0), sc.shape[0]
    if sc.dim() == want + 1:                   # paged
        if sc.shape[1] != page_size or (per_head and sc.shape[2] != H):
            raise ValueError("paged scale cache must be [pages, page_size(, H)]")
        return (sc.stride(0) * 4, sc.stride(1) * 4,
                sc.stride(2) * 4 if per_head else 0), sc.shape[0] * page_size
    raise ValueError("unsupported scale cache shape")


def store_kv_fp8_paged_dynamic(k, v, k_cache, v_cache, cache_loc, k_scale_cache, v_scale_cache,
                               per_head=False, page_size=16, size_limit=None, stream=None) -> None:
    """Fused e4m3fn quantise + paged store with per-token (or per token and
    head) scales computed in the kernel and written to the scale caches."""
    torch = _torch()
    _fp8_format(k_cache, v_cache, "e4m3fn", allowed=("e4m3fn",))
    dev = _device_of(k, v, k_cache, v_cache, cache_loc, k_scale_cache, v_scale_cache)
    if k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16:
        src = SRC_BF16
    elif k.dtype == torch.float16 and v.dtype == torch.float16:
        src = SRC_FP16
    else:
        raise TypeError("k and v must both be bfloat16 or both float16")
    H, D, slots, kcs = _cache_strides(k_cache, page_size)
    H2, D2, slots2, vcs = _cache_strides(v_cache, page_size)
    if (H, D, slots) != (H2, D2, slots2):
        raise ValueError("k_cache and v_cache shapes differ")
    kss, kslots = _scale_strides(k_scale_cache, per_head, H, page_size)
    vss, vslots = _scale_strides(v_scale_cache, per_head, H, page_size)
    if kslots != slots or vslots != slots:
        raise ValueError("scale caches must cover the same slots as the caches")
    ks = _input_strides(k, H, D)
    vs = _input_strides(v, H, D)
    T = k.shape[0]
    if v.shape[0] != T or cache_loc.dim() != 1 or cache_loc.shape[0] != T:
        raise ValueError("cache_loc must be [T] with T = k.shape[0] = v.shape[0]")
    limit = _size_limit(size_limit, slots)
    with torch.cuda.device(dev):
        st = kvstore_fp8_paged_dynamic(
            k.data_ptr(), v.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            cache_loc.data_ptr(), _idx_code(cache_loc), cache_loc.stride(0) if T else 1, src, H,
            D, ks[0], ks[1], vs[0], vs[1], kcs[0], kcs[1], kcs[2], vcs[0], vcs[1], vcs[2],
            k_scale_cache.data_ptr(), v_scale_cache.data_ptr(),
            SCALE_PER_TOKEN_HEAD if per_head else SCALE_PER_TOKEN, kss[0], kss[1], kss[2],
            vss[0], vss[1], vss[2], T, limit, page_size, _stream_handle(stream, dev))
    if st != OK:
        raise KVStoreError(st, "kvstore_fp8_paged_dynamic")


def take_error(out, stream=None):
    """Enqueue the graph-capturable error take: `out`, an int64 GPU tensor of
    two elements, receives (first_bad_token or -1, bad_count) when the stream
    reaches the call, and the flag is cleared.  Does not synchronise."""
    torch = _torch()
    dev = _device_of(out)
    if out.dtype != torch.int64 or out.numel() != 2 or not out.is_contiguous():
        raise TypeError("out must be a contiguous int64 GPU tensor of two elements")
    with torch.cuda.device(dev):
        st = kvstore_take_error(out.data_ptr(), _stream_handle(stream, dev))
    if st != OK:
        raise KVStoreError(st, "kvstore_take_error")


def check_error(stream=None, device=None):
    """(first_bad_token, bad_count) since the last check on `device` (default:
    the current device); (-1, 0) if none.  Synchronises the stream (default:
    that device's current stream)."""
    torch = _torch()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    with torch.cuda.device(dev):
        st, fb, bc = kvstore_check_error(_stream_handle(stream, dev))
    if st not in (OK, ERR_OOB):
        raise KVStoreError(st, "kvstore_check_error")
    return fb, bc
