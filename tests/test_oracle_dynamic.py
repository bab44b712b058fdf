"""Pins for the oracle's dynamic-scale FP8 store (CPU only).

Reading (the docstring of sglang "trtllm_fp8_kv_kernel.py" names per-token
scale computation as a step of the fused store; its code only applies a given
scale): per group (a token's K or V row, or one head of it) amax = max |x|
ignoring NaN; scale = max(amax / 448, 2^-126) in fp32 (the floor keeps
1 / scale finite); inv = 1 / scale in fp32 (the page's wrapper inverts a scale
the same way); codes are
e4m3fn(x * inv); the fp32 scale is stored beside the slot.

Pinned by an independent float32 reference (numpy division and multiply,
brute-force nearest-code search), closed-form properties, and edge groups.
"""
import numpy as np
import pytest

import kvgen
import oracle
from tests import _ref


def dyn_case(tokens=300, pages=8, src="bf16"):
    c = kvgen.workload(4, tokens=tokens, slots=pages * 64)
    c.src_dtype = src
    return c


@pytest.mark.parametrize("per_head", [False, True])
@pytest.mark.parametrize("src", ["bf16", "fp16"])
def test_matches_float32_reference(per_head, src):
    c = dyn_case(src=src)
    kc, vc, ks, vs, st = oracle.run_case_dynamic(c, per_head)
    assert st == (c.num_tokens, -1, 0)
    idx = c.indices.astype(np.int64)
    for cache, scales, src_bits in ((kc, ks, c.k), (vc, vs, c.v)):
        codes, sc = _ref.dynamic_expected(src_bits, c.src_dtype, c.num_heads, c.head_dim, per_head)
        np.testing.assert_array_equal(cache[idx], codes)
        np.testing.assert_array_equal(scales[idx], sc.view(np.uint32))
        untouched = np.ones(c.slots, dtype=bool)
        untouched[idx] = False
        assert np.all(cache[untouched] == 0xFF) and np.all(scales[untouched] == 0xFFFFFFFF)


def test_reference_distinguishes_inverse_forms():
    # 1 / (amax / 448) and 448 / amax round differently for some groups, so
    # the reference above would catch a kernel or oracle using the other form.
    c = dyn_case(tokens=300)
    x = _ref.src_bits_to_f32(c.k, "bf16").reshape(300, 8, 128)
    amax = np.abs(x).max(axis=2).astype(np.float32)
    a = (np.float32(1) / (amax / np.float32(448))).astype(np.float32)
    b = (np.float32(448) / amax).astype(np.float32)
    assert np.count_nonzero(a != b) > 10


@pytest.mark.parametrize("per_head", [False, True])
def test_largest_element_encodes_to_448(per_head):
    c = dyn_case(tokens=200)
    kc, _, ks, _, _ = oracle.run_case_dynamic(c, per_head)
    idx = c.indices.astype(np.int64)
    x = _ref.src_bits_to_f32(c.k, "bf16").reshape(200, 1 if not per_head else 8, -1)
    codes = kc[idx].reshape(x.shape)
    arg = np.abs(x).argmax(axis=2)
    top = np.take_along_axis(codes, arg[:, :, None], axis=2)[:, :, 0]
    assert np.all((top & 0x7F) == 0x7E)
    # scale * 448 gives back amax to within one float32 ulp
    amax = np.abs(x).max(axis=2)
    back = ks[idx].view(np.float32).reshape(amax.shape) * np.float32(448)
    assert np.all(np.abs(back - amax) <= np.spacing(amax.astype(np.float32)))


def test_per_token_scale_is_max_of_head_scales():
    c = dyn_case(tokens=100)
    _, _, ks_tok, _, _ = oracle.run_case_dynamic(c, False)
    _, _, ks_head, _, _ = oracle.run_case_dynamic(c, True)
    idx = c.indices.astype(np.int64)
    np.testing.assert_array_equal(ks_tok[idx, 0].view(np.float32),
                                  ks_head[idx].view(np.float32).max(axis=1))


def test_edge_groups():
    # token 0: all zeros; 1: one NaN among normals; 2: an infinity; 3: tiny
    # values (amax / 448 below the smallest normal); 4: negative zeros only
    c = dyn_case(tokens=8, pages=1)
    f = lambda vals: kvgen._round_f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))
    c.k[0, :] = 0
    c.k[1, 5] = 0x7FC1                     # NaN
    c.k[2, 7] = 0xFF80                     # -inf
    c.k[3, :] = f(np.full(1024, 1e-39))    # denormal-range bf16
    c.k[4, :] = 0x8000
    kc, _, ks, _, st = oracle.run_case_dynamic(c, False)
    assert st[0] == 8
    idx = c.indices.astype(np.int64)
    sc = ks[idx, 0].view(np.float32)
    tiny = np.float32(2.0 ** -126)
    assert sc[0] == tiny and np.all(kc[idx[0]] == 0x00)
    assert np.all(kc[idx[4]] == 0x80) and sc[4] == tiny
    x1 = _ref.bf16_bits_to_f32(c.k[1])
    assert sc[1] == np.float32(np.nanmax(np.abs(x1))) / np.float32(448)
    assert kc[idx[1], 5] == 0x7F
    assert sc[2] == np.inf
    assert kc[idx[2], 7] == 0xFF            # -inf * 0: the negative default NaN
    assert np.all(np.delete(kc[idx[2]], 7) & 0x7F == 0)
    assert sc[3] == tiny                   # amax / 448 < 2^-126: floored
    assert np.all(kc[idx[3]] != 0xFF) and np.all(kc[idx[3]] != 0x7F)
    codes, scales = _ref.dynamic_expected(c.k, "bf16", 8, 128, False)
    np.testing.assert_array_equal(kc[idx], codes)
    np.testing.assert_array_equal(sc, scales[:, 0])
