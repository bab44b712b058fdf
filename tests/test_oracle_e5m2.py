"""Pins for the oracle's e5m2 encoding and store (CPU only).

The page's unfused path (sglang "trtllm_fp8_kv_kernel.py",
_naive_fp8_set_kv_buffer) stores into float8_e5m2 as well as float8_e4m3fn
caches.  The encoding is written from the e5m2 definition with the same
reading as e4m3fn: round to nearest even, saturate to +-57344, NaN keeps its
sign.  Pinned by hand-derived values, a brute-force nearest-value search over
the decoded e5m2 table for every bf16 and fp16 pattern under each scale and
a million random fp32 values, and torch's own float8_e5m2 cast where it does
not overflow.
"""
import os

import numpy as np
import pytest
import torch

import kvgen
import oracle
from tests import _ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e5m2_pins.txt")
ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
INVS = [None, kvgen.INV_K_BITS, kvgen.INV_V_BITS]


def read_pins():
    ys, codes = [], []
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            a, b = line.split()[:2]
            ys.append(int(a, 16))
            codes.append(int(b, 16))
    return np.array(ys, dtype=np.uint32).view(np.float32), np.array(codes, dtype=np.uint8)


def test_golden_pins():
    y, want = read_pins()
    np.testing.assert_array_equal(oracle.e5m2(y), want)
    np.testing.assert_array_equal(_ref.nearest_e5m2(y), want)


def test_table_closed_form():
    t = _ref.TABLE_E5M2
    assert t.size == 124 and t[0] == 0 and t[-1] == 57344.0 and np.all(np.diff(t) > 0)
    assert t[4] == 2.0 ** -14 and t[0x3C] == 1.0


@pytest.mark.parametrize("src", ["bf16", "fp16"])
@pytest.mark.parametrize("inv", INVS, ids=["noscale", "inv_k", "inv_v"])
def test_exhaustive_against_nearest_value_search(src, inv):
    got = oracle.quantize(ALL16, src, inv, fmt="e5m2")
    want = _ref.expected_codes(ALL16, src, inv, fmt="e5m2")
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first 0x{int(ALL16[bad[0]]):04x}"


def test_random_fp32_against_nearest_value_search():
    rng = np.random.Generator(np.random.PCG64(13))
    bits = rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    near = rng.integers(0x36000000, 0x48000000, 1 << 19, dtype=np.uint64).astype(np.uint32)
    near |= rng.integers(0, 2, near.size, dtype=np.uint64).astype(np.uint32) << 31
    y = np.concatenate([bits, near]).view(np.float32)
    np.testing.assert_array_equal(oracle.e5m2(y), _ref.nearest_e5m2(y))


@pytest.mark.parametrize("src", ["bf16", "fp16"])
def test_torch_cast_where_it_does_not_overflow(src):
    x, y = _ref.scaled(ALL16, src, kvgen.INV_K_BITS)
    keep = np.isfinite(y) & (np.abs(y) <= 57344.0)
    t = torch.from_numpy(y[keep]).to(torch.float8_e5m2).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.quantize(ALL16, src, kvgen.INV_K_BITS, fmt="e5m2")[keep], t)
    assert keep.sum() > 30000


def test_store_layout_matches_e4m3_store_with_e5m2_codes():
    # The e5m2 store writes the same slots as the e4m3fn store; only codes differ.
    c = kvgen.workload(4, tokens=200, slots=8 * 64)
    kc, vc, st = oracle.run_case(c, fmt="e5m2")
    assert st == (200, -1, 0)
    idx = c.indices.astype(np.int64)
    np.testing.assert_array_equal(kc[idx], _ref.expected_codes(c.k, "bf16", c.inv_k_bits, "e5m2"))
    np.testing.assert_array_equal(vc[idx], _ref.expected_codes(c.v, "bf16", c.inv_v_bits, "e5m2"))
    untouched = np.ones(c.slots, dtype=bool)
    untouched[idx] = False
    assert np.all(kc[untouched] == 0xFF)
