"""GPU parity of the e5m2 fused paged store against the CPU oracle.

Every 16-bit bf16 / fp16 input pattern under each inverse scale (including
the edge scales), the FP8 workload at full size, and a padded layout; every
byte of both caches compared.
"""
import numpy as np
import pytest
import torch

import fp8_kv_quantization_amd as kv
import kvgen
import oracle
from tests import _ref
from tests._gpu import DEV, assert_cache_equal, check_flag, run_fp8, sentinel_cache, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


SCALES = {"none": None, "inv_k": kvgen.INV_K_BITS, "inv_v": kvgen.INV_V_BITS, "zero": 0x00000000,
          "inf": 0x7F800000, "nan": 0xFFC00000, "neg": 0xBECCCCCD, "huge": 0x7F000000,
          "tiny": 0x00000003}


@pytest.mark.parametrize("src", ["bf16", "fp16"])
@pytest.mark.parametrize("scale", list(SCALES))
def test_e5m2_every_input_pattern(src, scale):
    case = kvgen.all_patterns_case(src, inv_k_bits=SCALES[scale], inv_v_bits=kvgen.INV_V_BITS)
    _say(f"e5m2 all patterns {src} scale={scale}")
    kc = sentinel_cache(case.slots, case.row_elems)
    vc = sentinel_cache(case.slots, case.row_elems)
    assert run_fp8(case, kc, vc, fmt="e5m2") == kv.OK
    okc, ovc, _ = oracle.run_case(case, fmt="e5m2")
    got = kc.cpu().numpy()[:64].reshape(-1)
    want = okc[:64].reshape(-1)
    bad = np.nonzero(got != want)[0]
    if bad.size:
        pats = case.k.reshape(-1)[bad[:8]]
        raise AssertionError(f"{bad.size} patterns differ; e.g. " + ", ".join(
            f"0x{int(p):04x}->got 0x{int(g):02x} want 0x{int(w):02x}"
            for p, g, w in zip(pats, got[bad[:8]], want[bad[:8]])))
    assert_cache_equal(vc, ovc, "v_cache")
    np.testing.assert_array_equal(want, _ref.expected_codes(case.k, src, SCALES[scale], "e5m2").reshape(-1))


def test_e5m2_workload_full_size():
    c = kvgen.workload(4)
    _say("e5m2 full size")
    kc = sentinel_cache(c.slots, c.row_elems)
    vc = sentinel_cache(c.slots, c.row_elems)
    assert run_fp8(c, kc, vc, fmt="e5m2") == kv.OK
    assert check_flag() == (kv.OK, -1, 0)
    okc, ovc, st = oracle.run_case(c, fmt="e5m2")
    assert st == (c.num_tokens, -1, 0)
    assert_cache_equal(kc, okc, "k_cache")
    assert_cache_equal(vc, ovc, "v_cache")


def test_e5m2_tensor_api_from_cache_dtype():
    c = kvgen.workload(4, tokens=300, slots=16 * 64)
    H, D, P = 8, 128, 64
    kc = sentinel_cache(c.slots, H * D)
    vc = sentinel_cache(c.slots, H * D)
    ik = to_dev(np.array([c.inv_k_bits], dtype=np.uint32).view(np.float32))
    iv = to_dev(np.array([c.inv_v_bits], dtype=np.uint32).view(np.float32))
    kv.store_kv_fp8_paged(to_dev(c.k).view(torch.bfloat16).view(-1, H, D),
                          to_dev(c.v).view(torch.bfloat16).view(-1, H, D),
                          kc.view(-1, P, H, D).view(torch.float8_e5m2),
                          vc.view(-1, P, H, D).view(torch.float8_e5m2), to_dev(c.indices),
                          page_size=P, inv_k_scale=ik, inv_v_scale=iv)
    okc, ovc, _ = oracle.run_case(c, fmt="e5m2")
    np.testing.assert_array_equal(kc.cpu().numpy(), okc)
    np.testing.assert_array_equal(vc.cpu().numpy(), ovc)
