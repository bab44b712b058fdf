"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments before launching anything (CPU only: no GPU work).

The argument rules follow include/kvstore.h.  Each rejected case changes one
argument of an otherwise valid call; the expected status shows the call
returned during validation.  These cases use fake device addresses, so they
run only where no GPU is visible: a validation slip there would be a failed
launch, never a stray kernel.
"""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvstore.h")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="module")
def kv():
    import fp8_kv_quantization_amd as kv
    return kv


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(kvstore_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(
        ["kvstore_copy", "kvstore_fp8_paged", "kvstore_fp8_paged_e5m2",
         "kvstore_fp8_paged_dynamic", "kvstore_check_error", "kvstore_take_error",
         "kvstore_strerror"])


def test_library_exports_every_declared_symbol(kv):
    lib = C.CDLL(kv.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", kv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kvstore_\w+)", out))
    assert set(declared_functions()) <= exported


def test_binding_names_match_the_abi(kv):
    for name in declared_functions():
        assert callable(getattr(kv, name))
        # the compiled binding, not a Python stand-in
        assert type(getattr(kv, name)).__name__ == "builtin_function_or_method", name


def test_binding_links_the_in_tree_library(kv):
    from fp8_kv_quantization_amd import _kvstore_py
    out = subprocess.run(["ldd", _kvstore_py.__file__], capture_output=True, text=True,
                         check=True).stdout
    assert "libkvstore.so" in out and "not found" not in out.split("libkvstore.so")[1].split("\n")[0]


def test_binding_argument_errors(kv):
    with pytest.raises(TypeError):
        kv.kvstore_copy(0, 0, 0)                       # too few arguments
    with pytest.raises(TypeError):
        kv.kvstore_copy(*([0] * 15))                   # too many
    with pytest.raises(OverflowError):
        kv.kvstore_copy(0, 0, 0, 0, 0, 0, 1, 16, 16, 16, 16, 1 << 32, 1)   # batch > 32 bits
    with pytest.raises(TypeError):
        kv.kvstore_copy("k", 0, 0, 0, 0, 0, 1, 16, 16, 16, 16, 1, 1)      # not an int
    assert kv.kvstore_copy(0, 0, 0, 0, 0, 0, 1, 16, 16, 16, 16, 0, 1, None) == kv.OK


def test_strerror_texts(kv):
    for st in (kv.OK, kv.ERR_NULL, kv.ERR_SHAPE, kv.ERR_ALIGN, kv.ERR_DTYPE, kv.ERR_HIP, kv.ERR_OOB):
        assert kv.kvstore_strerror(st) and kv.kvstore_strerror(st) != "unknown status"
    assert kv.kvstore_strerror(12345) == "unknown status"


A = 0x7F0000000000  # fake, 256-byte aligned device addresses (never dereferenced)

COPY_OK = dict(k=A, v=A + 0x100000, k_cache=A + 0x200000, v_cache=A + 0x300000,
               indices=A + 0x400000, idx_dtype=0, idx_stride=1, row_bytes=2048,
               k_stride_bytes=2048, v_stride_bytes=2048, cache_stride_bytes=2048, batch=16,
               size_limit=1024)

# Longest row per lane width: 65535 grid slices x 4 chunks x 64 lanes x VW bytes.
COPY_MAX_ROW = {vw: 65535 * 4 * 64 * vw for vw in (16, 8, 4)}
# Most elements per FP8 row: 2 x 65535 grid rows (K and V) hold 32767 slices of
# 2 waves' worth of 16-element units each.
FP8_MAX_ELEMS = 32767 * 2 * 64 * 16


def _fp8_wide(elems):
    """A one-head FP8 layout with `elems` elements per row (flat caches)."""
    return dict(num_heads=1, head_dim=elems, k_stride_token_bytes=2 * elems,
                v_stride_token_bytes=2 * elems, k_stride_head_bytes=0, v_stride_head_bytes=0,
                kc_stride_page_bytes=64 * elems, kc_stride_offset_bytes=elems,
                kc_stride_head_bytes=0, vc_stride_page_bytes=64 * elems,
                vc_stride_offset_bytes=elems, vc_stride_head_bytes=0)


COPY_BAD = [
    ("null_k", dict(k=0), -1),
    ("null_cache", dict(v_cache=0), -1),
    ("null_indices", dict(indices=0), -1),
    ("bad_idx_dtype", dict(idx_dtype=2), -4),
    ("row_zero", dict(row_bytes=0), -2),
    ("row_negative", dict(row_bytes=-16), -2),
    ("row_not_4", dict(row_bytes=2042, k_stride_bytes=2048, cache_stride_bytes=2048), -2),
    ("row_too_big", dict(row_bytes=1 << 31, cache_stride_bytes=1 << 31, k_stride_bytes=0,
                         v_stride_bytes=0), -2),
    ("cache_stride_below_row", dict(cache_stride_bytes=1024), -2),
    # rows over 65535 grid slices of 4 lane-vector chunks
    ("row_over_slices_16B_lanes", dict(row_bytes=COPY_MAX_ROW[16] + 16, k_stride_bytes=0,
                                       v_stride_bytes=0,
                                       cache_stride_bytes=COPY_MAX_ROW[16] + 16), -2),
    ("row_over_slices_4B_lanes", dict(row_bytes=COPY_MAX_ROW[4] + 4, k_stride_bytes=0,
                                      v_stride_bytes=0,
                                      cache_stride_bytes=COPY_MAX_ROW[4] + 4), -2),
    ("negative_k_stride", dict(k_stride_bytes=-2048), -2),
    ("size_limit_zero", dict(size_limit=0), -2),
    ("size_limit_overflow", dict(size_limit=1 << 62), -2),
    ("idx_stride_zero", dict(idx_stride=0), -2),
    ("idx_stride_huge", dict(idx_stride=1 << 62), -2),
    ("k_misaligned", dict(k=A + 2), -3),
    ("cache_misaligned", dict(k_cache=A + 1), -3),
    ("stride_misaligned", dict(k_stride_bytes=2050), -3),
    ("cache_stride_misaligned", dict(cache_stride_bytes=2054), -3),
    ("i32_index_misaligned", dict(indices=A + 2), -3),
    ("i64_index_misaligned", dict(indices=A + 4, idx_dtype=1), -3),
]

FP8_OK = dict(k=A, v=A + 0x100000, k_cache=A + 0x200000, v_cache=A + 0x300000,
              indices=A + 0x400000, idx_dtype=0, idx_stride=1, src_dtype=0, num_heads=8,
              head_dim=128, k_stride_token_bytes=2048, k_stride_head_bytes=256,
              v_stride_token_bytes=2048, v_stride_head_bytes=256, kc_stride_page_bytes=65536,
              kc_stride_offset_bytes=1024, kc_stride_head_bytes=128, vc_stride_page_bytes=65536,
              vc_stride_offset_bytes=1024, vc_stride_head_bytes=128, batch=16, size_limit=4096,
              page_size=64, inv_k_scale_ptr=A + 0x500000, inv_v_scale_ptr=None)

FP8_BAD = [
    ("null_v", dict(v=0), -1),
    ("bad_src_dtype", dict(src_dtype=7), -4),
    ("bad_idx_dtype", dict(idx_dtype=-1), -4),
    ("heads_zero", dict(num_heads=0), -2),
    ("head_dim_not_16", dict(head_dim=120), -2),
    ("head_dim_zero", dict(head_dim=0), -2),
    ("page_size_zero", dict(page_size=0), -2),
    ("size_limit_negative", dict(size_limit=-1), -2),
    ("negative_stride", dict(kc_stride_head_bytes=-128), -2),
    ("stride_misaligned", dict(v_stride_head_bytes=264), -3),
    ("cache_stride_misaligned", dict(vc_stride_offset_bytes=1032), -3),
    ("head_offsets_over_32bit", dict(kc_stride_head_bytes=1 << 30), -2),
    # (heads - 1) * head stride beyond int64: must not wrap into a passing value
    ("head_stride_product_overflow", dict(num_heads=1 << 20, head_dim=16,
                                          k_stride_head_bytes=1 << 50), -2),
    ("cache_head_stride_product_overflow", dict(num_heads=1 << 20, head_dim=16,
                                                vc_stride_head_bytes=(1 << 62) + 16), -2),
    # slot offset plus the in-slot head span beyond int64
    ("slot_plus_head_span_overflow", dict(size_limit=64, kc_stride_page_bytes=64 * ((1 << 57) - 16),
                                          kc_stride_offset_bytes=(1 << 57) - 16,
                                          kc_stride_head_bytes=1 << 27), -2),
    ("slot_offset_overflow", dict(kc_stride_page_bytes=1 << 60, size_limit=1 << 20), -2),
    ("scale_misaligned", dict(inv_k_scale_ptr=A + 2), -3),
    ("cache_misaligned", dict(v_cache=A + 8), -3),
    ("idx_stride_zero", dict(idx_stride=0), -2),
    ("row_over_slices", _fp8_wide(FP8_MAX_ELEMS + 16), -2),
]


def _copy_call(kv, **over):
    a = dict(COPY_OK, **over)
    return kv.kvstore_copy(a["k"], a["v"], a["k_cache"], a["v_cache"], a["indices"],
                           a["idx_dtype"], a["idx_stride"], a["row_bytes"], a["k_stride_bytes"],
                           a["v_stride_bytes"], a["cache_stride_bytes"], a["batch"],
                           a["size_limit"], None)


def _fp8_call(kv, _entry=None, **over):
    a = dict(FP8_OK, **over)
    return (_entry or kv.kvstore_fp8_paged)(*[a[n] for n in (
        "k", "v", "k_cache", "v_cache", "indices", "idx_dtype", "idx_stride", "src_dtype",
        "num_heads", "head_dim", "k_stride_token_bytes", "k_stride_head_bytes",
        "v_stride_token_bytes", "v_stride_head_bytes", "kc_stride_page_bytes",
        "kc_stride_offset_bytes", "kc_stride_head_bytes", "vc_stride_page_bytes",
        "vc_stride_offset_bytes", "vc_stride_head_bytes", "batch", "size_limit", "page_size",
        "inv_k_scale_ptr", "inv_v_scale_ptr")], None)


cpu_only = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses: CPU-only check")


@cpu_only
@pytest.mark.parametrize("name,over,status", COPY_BAD, ids=[c[0] for c in COPY_BAD])
def test_copy_rejects(kv, name, over, status):
    assert _copy_call(kv, **over) == status


@cpu_only
@pytest.mark.parametrize("name,over,status", FP8_BAD, ids=[c[0] for c in FP8_BAD])
def test_fp8_rejects(kv, name, over, status):
    assert _fp8_call(kv, **over) == status
    assert _fp8_call(kv, _entry=kv.kvstore_fp8_paged_e5m2, **over) == status


@cpu_only
def test_empty_batch_returns_ok_without_launch(kv):
    # batch == 0 is accepted even with NULL pointers: nothing is launched.
    assert _copy_call(kv, batch=0, k=0, v=0, k_cache=0, v_cache=0, indices=0) == kv.OK
    assert _fp8_call(kv, batch=0, k=0, v=0, k_cache=0, v_cache=0, indices=0) == kv.OK
    # but the type codes are still checked
    assert _copy_call(kv, batch=0, idx_dtype=5) == kv.ERR_DTYPE


@cpu_only
def test_valid_arguments_reach_the_runtime(kv):
    # With no GPU the launch itself fails: the call got past validation.
    assert _copy_call(kv) == kv.ERR_HIP
    assert _fp8_call(kv) == kv.ERR_HIP
    assert _fp8_call(kv, _entry=kv.kvstore_fp8_paged_e5m2) == kv.ERR_HIP
    # 8- and 4-byte aligned rows and pointers are accepted by the copy
    assert _copy_call(kv, row_bytes=2040, k=A + 8) == kv.ERR_HIP
    # the longest rows pass validation
    # (a row of 4 mod 16 bytes takes 4-byte lanes)
    for row in (COPY_MAX_ROW[16], COPY_MAX_ROW[4] - 12):
        assert _copy_call(kv, row_bytes=row, k_stride_bytes=0, v_stride_bytes=0,
                          cache_stride_bytes=row) == kv.ERR_HIP
    assert _fp8_call(kv, **_fp8_wide(FP8_MAX_ELEMS)) == kv.ERR_HIP
    assert _copy_call(kv, row_bytes=36, k_stride_bytes=36, v_stride_bytes=40,
                      cache_stride_bytes=36, v_cache=A + 0x300004) == kv.ERR_HIP


DYN_OK = dict(FP8_OK, k_scale_cache=A + 0x600000, v_scale_cache=A + 0x700000, granularity=1,
              ks_stride_page_bytes=64 * 32, ks_stride_offset_bytes=32, ks_stride_head_bytes=4,
              vs_stride_page_bytes=64 * 32, vs_stride_offset_bytes=32, vs_stride_head_bytes=4)

DYN_BAD = [
    ("null_scale_cache", dict(v_scale_cache=0), -1),
    ("bad_granularity", dict(granularity=2), -4),
    ("row_too_wide", dict(num_heads=40), -2),                 # 5120 elements > 4096
    ("head_not_pow2_per_head", dict(num_heads=3, head_dim=48, k_stride_token_bytes=2048,
                                    v_stride_token_bytes=2048, k_stride_head_bytes=96,
                                    v_stride_head_bytes=96, kc_stride_head_bytes=48,
                                    vc_stride_head_bytes=48), -2),
    ("head_too_wide_per_head", dict(num_heads=2, head_dim=2048, k_stride_head_bytes=4096,
                                    v_stride_head_bytes=4096, kc_stride_head_bytes=2048,
                                    vc_stride_head_bytes=2048, k_stride_token_bytes=8192,
                                    v_stride_token_bytes=8192), -2),
    ("scale_misaligned", dict(k_scale_cache=A + 0x600002), -3),
    ("scale_stride_misaligned", dict(vs_stride_offset_bytes=34), -3),
    ("scale_stride_negative", dict(ks_stride_head_bytes=-4), -2),
    ("scale_offset_overflow", dict(ks_stride_page_bytes=1 << 61, size_limit=1 << 20), -2),
    # offset + head terms each within int64, their sum not (must not wrap)
    ("scale_offset_sum_overflow", dict(size_limit=64, ks_stride_offset_bytes=(1 << 57) - 4,
                                       ks_stride_head_bytes=(1 << 60) - 4), -2),
    ("inherits_fp8_checks", dict(head_dim=120), -2),
]


def _dyn_call(kv, **over):
    a = dict(DYN_OK, **over)
    return kv.kvstore_fp8_paged_dynamic(*[a[n] for n in (
        "k", "v", "k_cache", "v_cache", "indices", "idx_dtype", "idx_stride", "src_dtype",
        "num_heads", "head_dim", "k_stride_token_bytes", "k_stride_head_bytes",
        "v_stride_token_bytes", "v_stride_head_bytes", "kc_stride_page_bytes",
        "kc_stride_offset_bytes", "kc_stride_head_bytes", "vc_stride_page_bytes",
        "vc_stride_offset_bytes", "vc_stride_head_bytes", "k_scale_cache", "v_scale_cache",
        "granularity", "ks_stride_page_bytes", "ks_stride_offset_bytes", "ks_stride_head_bytes",
        "vs_stride_page_bytes", "vs_stride_offset_bytes", "vs_stride_head_bytes", "batch",
        "size_limit", "page_size")], None)


@cpu_only
@pytest.mark.parametrize("name,over,status", DYN_BAD, ids=[c[0] for c in DYN_BAD])
def test_dynamic_rejects(kv, name, over, status):
    assert _dyn_call(kv, **over) == status


@cpu_only
def test_dynamic_valid_arguments_reach_the_runtime(kv):
    assert _dyn_call(kv) == kv.ERR_HIP
    assert _dyn_call(kv, granularity=0, num_heads=3, head_dim=48, k_stride_token_bytes=2048,
                     v_stride_token_bytes=2048, k_stride_head_bytes=96, v_stride_head_bytes=96,
                     kc_stride_head_bytes=48, vc_stride_head_bytes=48) == kv.ERR_HIP
    assert _dyn_call(kv, batch=0, k=0) == kv.OK


def test_take_error_rejects_before_launch(kv):
    assert kv.kvstore_take_error(None) == kv.ERR_NULL
    assert kv.kvstore_take_error(A + 4) == kv.ERR_ALIGN
