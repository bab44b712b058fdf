"""Pins for the oracle's element arithmetic (CPU only).

The oracle's fused-store element step is: decode bf16/fp16 -> fp32, multiply
by the fp32 inverse scale (sglang "trtllm_fp8_kv_kernel.py", _process_kv_tensor:
the block times inv_scale, then the cast to float8 e4m3), round to the nearest
e4m3fn value with ties to even and saturation to +-448.  Each step is pinned
against something other than the oracle itself:

* decoding: torch's bfloat16 and numpy's float16 conversions, every pattern;
* fp32 multiply: numpy's float32 multiply on random operands;
* encoding: a brute-force nearest-value search over the e4m3fn table decoded
  from the format definition, for every bf16 and every fp16 pattern under each
  of the three inverse scales, and for a million random fp32 patterns;
* torch's own float8_e4m3fn cast wherever it does not overflow;
* hand-derived closed-form values in tests/golden/e4m3fn_pins.txt.
"""
import os

import numpy as np
import pytest
import torch

import kvgen
import oracle
from tests import _ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_pins.txt")
INVS = [None, kvgen.INV_K_BITS, kvgen.INV_V_BITS]
ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def read_pins():
    ys, codes = [], []
    with open(GOLDEN) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            a, b = line.split()[:2]
            ys.append(int(a, 16))
            codes.append(int(b, 16))
    return (np.array(ys, dtype=np.uint32).view(np.float32), np.array(codes, dtype=np.uint8))


def test_golden_pins():
    y, expected = read_pins()
    assert y.size >= 30
    np.testing.assert_array_equal(oracle.e4m3fn(y), expected)


def test_bruteforce_reference_agrees_with_golden_pins():
    # The independent brute-force encoder is itself checked against the
    # hand-derived values, so a flaw in it cannot hide an oracle flaw.
    y, expected = read_pins()
    np.testing.assert_array_equal(_ref.nearest_e4m3fn(y), expected)


def test_table_closed_form():
    # 127 non-negative finite codes, strictly increasing, 0 .. 448.
    t = _ref.TABLE
    assert t.size == 127 and t[0] == 0.0 and t[-1] == 448.0
    assert np.all(np.diff(t) > 0)
    assert t[1] == 2.0 ** -9 and t[8] == 2.0 ** -6 and t[0x38] == 1.0


@pytest.mark.parametrize("src", ["bf16", "fp16"])
def test_decode_every_pattern(src):
    got = np.array([oracle.load().oracle_src_to_float(int(b), int(src == "fp16")) for b in ALL16],
                   dtype=np.float32)
    want = _ref.src_bits_to_f32(ALL16, src)
    nan = np.isnan(want)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    np.testing.assert_array_equal(np.signbit(got[nan]), np.signbit(want[nan]))


def test_fp32_multiply_matches_numpy():
    rng = np.random.Generator(np.random.PCG64(5))
    # operands spread over the whole exponent range, so products hit fp32
    # subnormals, normal values and overflow.
    a = (rng.standard_normal(20000) * 2.0 ** rng.integers(-140, 120, 20000)).astype(np.float32)
    b = (rng.standard_normal(20000) * 2.0 ** rng.integers(-20, 20, 20000)).astype(np.float32)
    lib = oracle.load()
    got = np.array([lib.oracle_mul_f32(float(x), float(y)) for x, y in zip(a, b)], dtype=np.float32)
    with np.errstate(all="ignore"):
        want = (a * b).astype(np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("src", ["bf16", "fp16"])
@pytest.mark.parametrize("inv", INVS, ids=["noscale", "inv_k", "inv_v"])
def test_exhaustive_against_nearest_value_search(src, inv):
    got = oracle.quantize(ALL16, src, inv)
    want = _ref.expected_codes(ALL16, src, inv)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first pattern 0x{int(ALL16[bad[0]]):04x}"


def test_random_fp32_against_nearest_value_search():
    # fp32 inputs with full 24-bit significands exercise the sticky bits that
    # bf16 inputs never set.
    rng = np.random.Generator(np.random.PCG64(11))
    bits = rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    # bias half of them into the e4m3fn range so rounding is exercised densely
    near = rng.integers(0x3A000000, 0x44000000, 1 << 19, dtype=np.uint64).astype(np.uint32)
    near |= (rng.integers(0, 2, near.size, dtype=np.uint64).astype(np.uint32) << 31)
    y = np.concatenate([bits, near]).view(np.float32)
    np.testing.assert_array_equal(oracle.e4m3fn(y), _ref.nearest_e4m3fn(y))


@pytest.mark.parametrize("src", ["bf16", "fp16"])
@pytest.mark.parametrize("inv", INVS, ids=["noscale", "inv_k", "inv_v"])
def test_torch_cast_where_it_does_not_overflow(src, inv):
    # torch's float8_e4m3fn cast is round-to-nearest-even; it differs from a
    # saturating cast only beyond +-448 (it returns NaN there), so compare
    # only finite |y| <= 448.
    x, y = _ref.scaled(ALL16, src, inv)
    keep = np.isfinite(y) & (np.abs(y) <= 448.0)
    t = torch.from_numpy(y[keep]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.quantize(ALL16, src, inv)[keep]
    np.testing.assert_array_equal(got, t)
    assert keep.sum() > 30000


def test_saturation_and_nan_cover_both_signs():
    y = np.array([449.0, -449.0, np.inf, -np.inf, np.nan, -np.nan, 1e38, -1e38], dtype=np.float32)
    y[5] = -np.abs(y[5])
    got = oracle.e4m3fn(y)
    np.testing.assert_array_equal(got, np.array([0x7E, 0xFE, 0x7E, 0xFE, 0x7F, 0xFF, 0x7E, 0xFE],
                                                dtype=np.uint8))


def test_codes_are_monotone_in_value():
    # Property of a correct rounding: a larger value never gets a smaller
    # code (positive half), across the whole finite fp32 range that matters.
    y = np.linspace(0.0, 500.0, 200001, dtype=np.float32)
    c = oracle.e4m3fn(y).astype(np.int32)
    assert np.all(np.diff(c) >= 0)
    assert c[0] == 0 and c[-1] == 0x7E


def test_nan_rules_of_the_product():
    # Reading: a NaN input is its own product (its sign kept, whatever the
    # scale); a NaN scale with a non-NaN input gives that scale's NaN; inf * 0
    # gives the negative default NaN, as torch's fp32 multiply on the CPU does.
    lib = oracle.load()
    f = lambda bits: float(np.array([bits], dtype=np.uint32).view(np.float32)[0])
    def sgn(x):
        return int(np.signbit(np.float32(x)))
    neg_nan, pos_nan = f(0xFFC00000), f(0x7FC00000)
    for x, inv, want_sign in ((neg_nan, 0.4, 1), (pos_nan, -0.4, 0), (neg_nan, pos_nan, 1),
                              (pos_nan, neg_nan, 0), (1.5, neg_nan, 1), (1.5, pos_nan, 0),
                              (float("inf"), 0.0, 1), (float("-inf"), 0.0, 1), (0.0, float("inf"), 1)):
        y = lib.oracle_mul_f32(x, inv)
        assert np.isnan(y) and sgn(y) == want_sign, (x, inv, y)
    codes = oracle.e4m3fn(np.array([neg_nan, pos_nan], dtype=np.float32))
    assert list(codes) == [0xFF, 0x7F]
    # the library routine this reading follows
    t = torch.tensor([float("inf"), float("-inf")]) * torch.tensor([0.0, 0.0])
    assert all(int(v) & 0xFFFFFFFF == 0xFFC00000 for v in t.view(torch.int32))
