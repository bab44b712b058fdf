"""The seeded input recipes (CPU): shapes, index structure, value
distribution, fixed scale bits and the algorithmic byte counts the bench
divides by, checked against the workload definitions written out by hand.

Byte counts per workload = K and V rows read (row bytes only, not stride
padding) + one index per token + K and V cache rows written (+ the two
4-byte inverse scales of the FP8 store)."""
import numpy as np
import pytest

import kvgen

# (tokens, row bytes read, index bytes, cache row bytes written, scale bytes)
EXPECTED = {
    1: (16, 2 * 64 * 2, 4, 2 * 64 * 2, 0),          # 16 tok, 2 heads x 64 bf16
    2: (256, 8 * 128 * 2, 8, 8 * 128 * 2, 0),       # 256 tok, 8 x 128 bf16, int64
    3: (32768, 8 * 128 * 2, 4, 8 * 128 * 2, 0),     # 32768 tok, int32
    4: (16384, 8 * 128 * 2, 4, 8 * 128, 8),         # bf16 in, one e4m3fn byte out
    5: (8192, 576 * 2, 8, 576 * 2, 0),              # 576 fp16 of a 640-element row
}
TOTALS = {1: 16_448, 2: 2_099_200, 3: 268_566_528, 4: 100_728_840, 5: 37_814_272}


def _f32_of(case, rows):
    """Decoded float32 values of the first `row_elems` columns."""
    bits = rows[:, :case.row_elems].astype(np.uint32)
    if case.src_dtype == kvgen.BF16:
        return (bits << 16).view(np.float32)
    return bits.astype(np.uint16).view(np.float16).astype(np.float32)


@pytest.fixture(scope="module")
def cases():
    return {n: kvgen.workload(n) for n in (1, 2, 3, 4, 5)}


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_algorithmic_bytes(cases, n):
    T, r, i, w, s = EXPECTED[n]
    assert 2 * T * r + T * i + 2 * T * w + s == TOTALS[n]
    assert cases[n].algorithmic_bytes() == TOTALS[n]


@pytest.mark.parametrize("n,slots,idx_dtype,stride", [(1, 256, np.int32, 128),
                                                      (2, 1 << 20, np.int64, 1024),
                                                      (3, 1 << 21, np.int32, 1024),
                                                      (4, 1 << 21, np.int32, 1024),
                                                      (5, 1 << 19, np.int64, 640)])
def test_shapes_and_unique_in_range_indices(cases, n, slots, idx_dtype, stride):
    c = cases[n]
    T = EXPECTED[n][0]
    assert c.k.shape == c.v.shape == (T, stride) and c.k.dtype == np.uint16
    assert c.indices.dtype == idx_dtype and c.indices.shape == (T,)
    assert c.slots == slots
    idx = c.indices.astype(np.int64)
    assert idx.min() >= 0 and idx.max() < slots
    assert np.unique(idx).size == T


@pytest.mark.parametrize("n,page", [(3, 16), (4, 64)])
def test_paged_runs(cases, n, page):
    """Consecutive runs of `page` tokens fill whole pages, in a shuffled page order."""
    idx = cases[n].indices.astype(np.int64)
    t = np.arange(idx.size)
    assert np.array_equal(idx % page, t % page)
    pages = (idx // page).reshape(-1, page)
    assert (pages == pages[:, :1]).all()
    order = pages[:, 0]
    assert np.unique(order).size == order.size
    assert not np.array_equal(order, np.sort(order))      # not in address order


def test_wide_rows_carry_poison_padding(cases):
    c = cases[5]
    assert (c.k[:, 576:] == kvgen.PAD_POISON).all() and (c.v[:, 576:] == kvgen.PAD_POISON).all()
    # the poison is an fp16 NaN, which a normal draw never produces
    assert np.isnan(np.array([kvgen.PAD_POISON], dtype=np.uint16).view(np.float16))[0]
    assert not np.isnan(_f32_of(c, c.k)).any()


@pytest.mark.parametrize("n", [2, 3, 5])
def test_values_are_standard_normal(cases, n):
    c = cases[n]
    x = np.concatenate([_f32_of(c, c.k).ravel(), _f32_of(c, c.v).ravel()]).astype(np.float64)
    assert abs(x.mean()) < 5 / np.sqrt(x.size)
    assert abs(x.std() - 1.0) < 0.01


def test_fp8_outliers(cases):
    """About 0.1% of elements scaled by 50: |x| > 10 is (practically) only an
    outlier whose base draw exceeded 0.2 in magnitude, a share of
    P(|z| > 0.2) = 0.8415 of them."""
    c = cases[4]
    x = np.concatenate([_f32_of(c, c.k).ravel(), _f32_of(c, c.v).ravel()])
    n = x.size
    expect = n * 0.001 * 0.8415
    hits = int((np.abs(x) > 10).sum())
    assert abs(hits - expect) < 6 * np.sqrt(expect), (hits, expect)
    assert np.abs(x).max() < 448          # the workload never saturates


def test_inverse_scale_bits():
    inv_k = np.float32(1.0) / np.float32(2.5)
    inv_v = np.float32(1.0) / np.float32(1.7)
    assert int(inv_k.view(np.uint32)) == kvgen.INV_K_BITS == 0x3ECCCCCD
    assert int(inv_v.view(np.uint32)) == kvgen.INV_V_BITS == 0x3F169696
    # the one-step double-precision reciprocal rounds differently for V
    assert int(np.float32(1.0 / 1.7).view(np.uint32)) == 0x3F169697


def test_seeded_and_deterministic():
    a, b = kvgen.workload(1), kvgen.workload(1)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    assert np.array_equal(a.indices, b.indices)
    assert a.seed == 1001
    other = kvgen.workload(1, seed=7)
    assert not np.array_equal(a.k, other.k)


@pytest.mark.parametrize("n,count", [(3, 8), (4, 8), (5, 16), (2, 4)])
def test_disjoint_index_sets(cases, n, count):
    c = cases[n]
    sets = kvgen.disjoint_index_sets(c, count)
    assert np.array_equal(sets[0], c.indices)
    allidx = np.concatenate([s.astype(np.int64) for s in sets])
    assert np.unique(allidx).size == count * c.num_tokens
    assert allidx.min() >= 0 and allidx.max() < c.slots
    page = c.extra.get("index_page", 1)
    if page > 1:
        t = np.arange(c.num_tokens)
        for s in sets:
            assert np.array_equal(s.astype(np.int64) % page, t % page)


def _check_runs(case, s):
    """Index array s keeps the case's scheme: tokens t of one run go to
    consecutive slots of one whole run, each run used once."""
    run = case.extra["index_page"]
    t = np.arange(case.num_tokens)
    s = s.astype(np.int64)
    assert np.array_equal(s % run, t % run)
    starts = (s // run)[::run]
    assert np.array_equal(s // run, np.repeat(starts, run)[:case.num_tokens])
    assert np.unique(starts).size == starts.size


@pytest.mark.parametrize("pattern", kvgen.DEST_PATTERNS)
def test_pattern_index_sets(cases, pattern):
    c = cases[3]
    sets = kvgen.pattern_index_sets(c, pattern, 8)
    allidx = np.concatenate([s.astype(np.int64) for s in sets])
    assert np.unique(allidx).size == 8 * c.num_tokens
    assert allidx.min() >= 0 and allidx.max() < c.slots
    assert all(s.dtype == c.indices.dtype for s in sets)
    T = c.num_tokens
    if pattern == "contiguous":
        for k, s in enumerate(sets):
            assert np.array_equal(s, np.arange(k * T, (k + 1) * T))
    elif pattern == "runs16_in_64MiB":
        for k, s in enumerate(sets):
            _check_runs(c, s)
            # set k fills its own 64 MiB extent exactly
            assert np.array_equal(np.sort(s.astype(np.int64)), np.arange(k * T, (k + 1) * T))
            assert T * c.row_bytes == 64 << 20
    elif pattern == "workload":
        assert np.array_equal(sets[0], c.indices)
        for s in sets:
            _check_runs(c, s)


@pytest.mark.parametrize("mib", kvgen.EXTENT_MIB)
def test_extent_index_sets(cases, mib):
    c = cases[3]
    E = (mib << 20) // c.row_bytes                  # slots per extent
    sets = kvgen.extent_index_sets(c, mib << 20, 8)
    allidx = np.concatenate([s.astype(np.int64) for s in sets])
    assert np.unique(allidx).size == 8 * c.num_tokens
    assert allidx.min() >= 0 and allidx.max() < c.slots
    own = 8 * E <= c.slots and E < 8 * c.num_tokens
    for k, s in enumerate(sets):
        _check_runs(c, s)
        lo, hi = (k * E, (k + 1) * E) if own else (0, E)
        assert s.min() >= lo and s.max() < hi, (mib, k)
    # the runs spread over the extent: the written slots span most of it
    span = allidx.max() - allidx.min() + 1 if not own else sets[0].max() - sets[0].min() + 1
    assert span > 0.9 * E


def test_extent_index_sets_refuses_what_does_not_fit(cases):
    c = cases[3]
    with pytest.raises(ValueError):
        kvgen.extent_index_sets(c, 32 << 20, 8)    # smaller than one set's runs
    with pytest.raises(ValueError):
        kvgen.extent_index_sets(c, 8 << 30, 8)     # larger than the cache
