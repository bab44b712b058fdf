"""Pins for the oracle's store semantics (CPU only).

Copy: sglang "kvcache.cuh", store_kvcache -- token t's K and V rows land
byte-for-byte in cache row indices[t]; an index outside [0, size_limit) is
rejected (the page asserts; here the row is skipped and counted).
Fused FP8 paged store: sglang "trtllm_fp8_kv_kernel.py",
_fused_fp8_set_kv_buffer_kernel -- page = loc // page_size,
offset = loc % page_size, byte at [page, offset, head, dim]; the page's
fused_fp8_set_kv_buffer wrapper accepts a flat [slots, H, D] cache whose page
stride is page_size slot strides, and its naive fallback writes through
index_put at (page_ids, page_offsets).

Pinned by: a pure-Python brute-force copy, numpy fancy-index round trips,
sentinel-filled caches with guard rows past size_limit, token-permutation
invariance, paged == flat equivalence on padded layouts, and torch's own
index_put with its float8_e4m3fn cast for the FP8 store.
"""
import numpy as np
import pytest
import torch

import kvgen
import oracle
from tests import _ref


def as_bytes(a16: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a16).view(np.uint8)


def small_copy_case(n, tokens, slots):
    return kvgen.workload(n, tokens=tokens, slots=slots)


# ---------------------------------------------------------------------------
# Copy
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,tokens,slots", [(1, None, None), (2, 40, 512), (5, 33, 256)])
def test_copy_matches_python_bruteforce(n, tokens, slots):
    c = small_copy_case(n, tokens, slots)
    kb, vb = as_bytes(c.k), as_bytes(c.v)
    guard = 3
    kc = np.full((c.slots + guard, c.row_bytes), 0xFF, dtype=np.uint8)
    vc = np.full_like(kc, 0xFF)
    st = oracle.copy(kb, vb, kc, vc, c.indices, row_bytes=c.row_bytes,
                     k_stride=c.in_stride_bytes, v_stride=c.in_stride_bytes,
                     cache_stride=c.row_bytes, size_limit=c.slots)
    bk, bv, bad = _ref.copy_bruteforce(kb.tobytes(), vb.tobytes(), c.indices, c.row_bytes,
                                       c.in_stride_bytes, c.in_stride_bytes, c.slots + guard,
                                       c.row_bytes, c.slots)
    assert st == (c.num_tokens, -1, 0) and bad == []
    np.testing.assert_array_equal(kc, bk)
    np.testing.assert_array_equal(vc, bv)


@pytest.mark.parametrize("row,stride", [(4, 4), (12, 20), (36, 44), (8, 8), (24, 40), (100, 104)])
def test_copy_rows_of_four_byte_multiples_match_bruteforce(row, stride):
    # The copy page accepts any row size that is a multiple of 4 bytes
    # (kvcache.cuh, copy_kv_warp: vectors of 16, 8 or 4 bytes).
    rng = np.random.Generator(np.random.PCG64(row))
    T, slots = 37, 64
    kb = rng.integers(0, 256, (T, stride), dtype=np.uint8)
    vb = rng.integers(0, 256, (T, stride), dtype=np.uint8)
    idx = rng.permutation(slots)[:T].astype(np.int32)
    kc = np.full((slots, row), 0xFF, dtype=np.uint8)
    vc = np.full_like(kc, 0xFF)
    st = oracle.copy(kb, vb, kc, vc, idx, row_bytes=row, k_stride=stride, v_stride=stride,
                     cache_stride=row, size_limit=slots)
    bk, bv, bad = _ref.copy_bruteforce(kb.tobytes(), vb.tobytes(), idx, row, stride, stride,
                                       slots, row, slots)
    assert st == (T, -1, 0) and bad == []
    np.testing.assert_array_equal(kc, bk)
    np.testing.assert_array_equal(vc, bv)


@pytest.mark.parametrize("n,tokens,slots", [(2, 300, 4096), (3, 1000, 4096), (5, 257, 2048)])
def test_copy_roundtrip_and_sentinel(n, tokens, slots):
    c = small_copy_case(n, tokens, slots)
    kc, vc, st = oracle.run_case(c)
    assert st == (c.num_tokens, -1, 0)
    R = c.row_bytes
    idx = c.indices.astype(np.int64)
    np.testing.assert_array_equal(kc[idx], as_bytes(c.k)[:, :R])
    np.testing.assert_array_equal(vc[idx], as_bytes(c.v)[:, :R])
    untouched = np.ones(c.slots, dtype=bool)
    untouched[idx] = False
    assert np.all(kc[untouched] == 0xFF) and np.all(vc[untouched] == 0xFF)


def test_copy_strided_padding_never_reaches_cache():
    c = small_copy_case(5, 300, 1024)
    assert c.in_stride_elems == 640 and c.row_elems == 576
    assert np.all(c.k[:, 576:] == kvgen.PAD_POISON)
    kc, vc, _ = oracle.run_case(c)
    for cache in (kc, vc):
        assert not np.any(cache.view(np.uint16) == kvgen.PAD_POISON)


def test_copy_token_order_does_not_matter():
    c = small_copy_case(3, 500, 2048)
    kc1, vc1, _ = oracle.run_case(c)
    p = np.random.Generator(np.random.PCG64(3)).permutation(c.num_tokens)
    c.k, c.v, c.indices = c.k[p].copy(), c.v[p].copy(), c.indices[p].copy()
    kc2, vc2, _ = oracle.run_case(c)
    np.testing.assert_array_equal(kc1, kc2)
    np.testing.assert_array_equal(vc1, vc2)


@pytest.mark.parametrize("idx_dtype", [np.int32, np.int64])
def test_copy_out_of_bounds_rows_are_skipped_and_counted(idx_dtype):
    c = small_copy_case(2, 64, 256)
    limit = 200                       # caches hold 256 rows; rows >= 200 are guard rows
    idx = np.random.Generator(np.random.PCG64(9)).permutation(limit)[:64].astype(idx_dtype)
    info = np.iinfo(idx_dtype)
    bad_at = {5: -1, 17: limit, 40: info.max, 63: info.min, 41: limit + 1}
    for t, val in bad_at.items():
        idx[t] = val
    R = c.row_bytes
    kc = np.full((256, R), 0xFF, dtype=np.uint8)
    vc = np.full_like(kc, 0xFF)
    n, first, count = oracle.copy(as_bytes(c.k), as_bytes(c.v), kc, vc, idx, row_bytes=R,
                                  k_stride=R, v_stride=R, cache_stride=R, size_limit=limit)
    assert (n, first, count) == (64 - len(bad_at), 5, len(bad_at))
    assert np.all(kc[limit:] == 0xFF) and np.all(vc[limit:] == 0xFF)
    good = [t for t in range(64) if t not in bad_at]
    np.testing.assert_array_equal(kc[idx[good].astype(np.int64)], as_bytes(c.k)[good])
    np.testing.assert_array_equal(vc[idx[good].astype(np.int64)], as_bytes(c.v)[good])


def test_copy_last_valid_slot_and_index_stride():
    c = small_copy_case(1, None, None)
    idx = c.indices.copy()
    last = c.slots - 1
    if last in idx:
        idx[list(idx).index(last)] = idx[3]
    idx[3] = last
    strided = np.full(idx.size * 3, -7, dtype=idx.dtype)   # junk between the used entries
    strided[::3] = idx
    R = c.row_bytes
    a = [np.full((c.slots, R), 0xFF, dtype=np.uint8) for _ in range(4)]
    s1 = oracle.copy(as_bytes(c.k), as_bytes(c.v), a[0], a[1], idx, row_bytes=R, k_stride=R,
                     v_stride=R, cache_stride=R, size_limit=c.slots)
    s2 = oracle.copy(as_bytes(c.k), as_bytes(c.v), a[2], a[3], strided, row_bytes=R,
                     k_stride=R, v_stride=R, cache_stride=R, size_limit=c.slots, idx_stride=3,
                     batch=idx.size)
    assert s1 == s2 == (idx.size, -1, 0)
    np.testing.assert_array_equal(a[0], a[2])
    np.testing.assert_array_equal(a[1], a[3])
    np.testing.assert_array_equal(a[0][last], as_bytes(c.k)[3])


def test_copy_empty_batch_is_a_no_op():
    c = small_copy_case(1, None, None)
    R = c.row_bytes
    kc = np.full((c.slots, R), 0xFF, dtype=np.uint8)
    vc = np.full_like(kc, 0xFF)
    st = oracle.copy(as_bytes(c.k), as_bytes(c.v), kc, vc, c.indices, row_bytes=R, k_stride=R,
                     v_stride=R, cache_stride=R, size_limit=c.slots, batch=0)
    assert st == (0, -1, 0) and np.all(kc == 0xFF) and np.all(vc == 0xFF)


# ---------------------------------------------------------------------------
# Fused FP8 paged store
# ---------------------------------------------------------------------------

def fp8_small(tokens=200, pages=32, src="bf16", page_size=64, inv=True, seed=None):
    c = kvgen.workload(4, tokens=tokens, slots=pages * 64, seed=seed)
    if src == "fp16":
        c.src_dtype = "fp16"        # same bit patterns, read as (finite) fp16 values
    if not inv:
        c.inv_k_bits = c.inv_v_bits = None
    if page_size != 64:
        c.page_size = page_size
        c.slots = (c.slots // page_size) * page_size
        c.indices = c.indices[c.indices < c.slots].copy()
        c.k, c.v = c.k[:c.indices.size].copy(), c.v[:c.indices.size].copy()
        c.num_tokens = c.indices.size
    return c


@pytest.mark.parametrize("src,inv", [("bf16", True), ("bf16", False), ("fp16", True)])
def test_fp8_each_element_is_the_nearest_code(src, inv):
    c = fp8_small(src=src, inv=inv)
    kc, vc, st = oracle.run_case(c)
    assert st == (c.num_tokens, -1, 0)
    idx = c.indices.astype(np.int64)
    want_k = _ref.expected_codes(c.k, c.src_dtype, c.inv_k_bits)
    want_v = _ref.expected_codes(c.v, c.src_dtype, c.inv_v_bits)
    np.testing.assert_array_equal(kc[idx], want_k)
    np.testing.assert_array_equal(vc[idx], want_v)
    untouched = np.ones(c.slots, dtype=bool)
    untouched[idx] = False
    assert np.all(kc[untouched] == 0xFF) and np.all(vc[untouched] == 0xFF)


def test_fp8_matches_torch_index_put_path():
    # The page's unfused fallback: cast with torch, then index_put at
    # (loc // page_size, loc % page_size) into a 4-D cache.  It scales in fp32
    # here (the fused kernel's arithmetic) so only the layout and the cast are
    # compared; its torch cast is exact for these values (all below 448).
    c = fp8_small(tokens=300, pages=16)
    H, D, P = c.num_heads, c.head_dim, c.page_size
    kc, vc, _ = oracle.run_case(c)
    loc = torch.from_numpy(c.indices.astype(np.int64))
    for src, inv_bits, got in ((c.k, c.inv_k_bits, kc), (c.v, c.inv_v_bits, vc)):
        x = torch.from_numpy(_ref.bf16_bits_to_f32(src))
        inv = torch.tensor(np.array([inv_bits], dtype=np.uint32).view(np.float32)[0])
        y = (x * inv).view(-1, H, D)
        assert float(y.abs().max()) < 448.0
        q = y.to(torch.float8_e4m3fn).view(torch.uint8)
        cache4 = torch.full((c.slots // P, P, H, D), 0xFF, dtype=torch.uint8)
        cache4[loc // P, loc % P] = q
        np.testing.assert_array_equal(got.reshape(-1), cache4.numpy().reshape(-1))


def test_fp8_paged_layout_equals_flat_layout():
    # Same logical store into (a) a flat [slots, H, D] cache and (b) a padded
    # 4-D [pages, P, H, D] cache (extra bytes after every head and every page).
    c = fp8_small(tokens=150, pages=8, page_size=48)
    H, D, P = c.num_heads, c.head_dim, c.page_size
    row = H * D
    flat_k = np.full((c.slots, row), 0xFF, dtype=np.uint8)
    flat_v = np.full_like(flat_k, 0xFF)
    kw = dict(src_dtype=c.src_dtype, num_heads=H, head_dim=D, k_strides=(row * 2, D * 2),
              v_strides=(row * 2, D * 2), size_limit=c.slots, page_size=P,
              inv_k_bits=c.inv_k_bits, inv_v_bits=c.inv_v_bits)
    oracle.fp8_paged(c.k, c.v, flat_k, flat_v, c.indices, kc_strides=(P * row, row, D),
                     vc_strides=(P * row, row, D), **kw)
    sh = D + 32
    so = H * sh + 64
    sp = P * so + 4096
    pages = c.slots // P
    pk = np.full(pages * sp, 0xFF, dtype=np.uint8)
    pv = np.full_like(pk, 0xFF)
    oracle.fp8_paged(c.k, c.v, pk, pv, c.indices, kc_strides=(sp, so, sh), vc_strides=(sp, so, sh),
                     **kw)
    for flat, paged in ((flat_k, pk), (flat_v, pv)):
        view = np.lib.stride_tricks.as_strided(paged, shape=(pages, P, H, D),
                                               strides=(sp, so, sh, 1))
        np.testing.assert_array_equal(view.reshape(c.slots, row), flat)
        # padding bytes untouched
        mask = np.ones(pages * sp, dtype=bool)
        off = (np.arange(pages)[:, None, None, None] * sp + np.arange(P)[None, :, None, None] * so
               + np.arange(H)[None, None, :, None] * sh + np.arange(D)[None, None, None, :])
        mask[off.ravel()] = False
        assert np.all(paged[mask] == 0xFF)


def test_fp8_strided_input_heads():
    # Input heads not contiguous: [T, H, D] with a padded head stride.
    c = fp8_small(tokens=100, pages=4)
    H, D = c.num_heads, c.head_dim
    sh = D + 8                                     # elements
    buf_k = np.full((c.num_tokens, H, sh), kvgen.PAD_POISON, dtype=np.uint16)
    buf_v = np.full_like(buf_k, kvgen.PAD_POISON)
    buf_k[:, :, :D] = c.k.reshape(-1, H, D)
    buf_v[:, :, :D] = c.v.reshape(-1, H, D)
    row = H * D
    kc = np.full((c.slots, row), 0xFF, dtype=np.uint8)
    vc = np.full_like(kc, 0xFF)
    oracle.fp8_paged(buf_k, buf_v, kc, vc, c.indices, src_dtype="bf16", num_heads=H, head_dim=D,
                     k_strides=(H * sh * 2, sh * 2), v_strides=(H * sh * 2, sh * 2),
                     kc_strides=(64 * row, row, D), vc_strides=(64 * row, row, D),
                     size_limit=c.slots, page_size=64, inv_k_bits=c.inv_k_bits,
                     inv_v_bits=c.inv_v_bits)
    kc2, vc2, _ = oracle.run_case(c)
    np.testing.assert_array_equal(kc, kc2)
    np.testing.assert_array_equal(vc, vc2)


def test_fp8_one_scale_given_other_tensor_unscaled():
    c = fp8_small(tokens=64, pages=2)
    c.inv_v_bits = None
    kc, vc, _ = oracle.run_case(c)
    idx = c.indices.astype(np.int64)
    np.testing.assert_array_equal(kc[idx], _ref.expected_codes(c.k, "bf16", kvgen.INV_K_BITS))
    np.testing.assert_array_equal(vc[idx], _ref.expected_codes(c.v, "bf16", None))


def test_fp8_out_of_bounds_rows_are_skipped_and_counted():
    c = fp8_small(tokens=128, pages=4)            # 256 slots
    limit = 192
    idx = np.random.Generator(np.random.PCG64(2)).permutation(limit)[:128].astype(np.int32)
    idx[0] = limit
    idx[77] = -5
    c.indices = idx
    row = c.row_elems
    kc = np.full((256, row), 0xFF, dtype=np.uint8)
    vc = np.full_like(kc, 0xFF)
    H, D = c.num_heads, c.head_dim
    st = oracle.fp8_paged(c.k, c.v, kc, vc, idx, src_dtype="bf16", num_heads=H, head_dim=D,
                          k_strides=(row * 2, D * 2), v_strides=(row * 2, D * 2),
                          kc_strides=(64 * row, row, D), vc_strides=(64 * row, row, D),
                          size_limit=limit, page_size=64, inv_k_bits=c.inv_k_bits,
                          inv_v_bits=c.inv_v_bits)
    assert st == (126, 0, 2)
    assert np.all(kc[limit:] == 0xFF) and np.all(vc[limit:] == 0xFF)


def test_k_and_v_layouts_are_independent():
    """K and V inputs, caches and scale caches each at their own strides: a V
    that borrowed one of K's strides would read or write the wrong bytes
    (copy, fused FP8 and per-head dynamic-scale stores)."""
    from tests import _battery
    lib = oracle.load()
    assert _battery._copy(lib)
    assert _battery._fp8(lib)
    assert _battery._dynamic_layouts(lib)
