"""Seeded randomized parity: every store entry point over random layouts.

Each trial draws (from a fixed seed) the operation, token count, heads and
head size, input and cache paddings, page size, index type and stride, scales
and a few out-of-range indices (tests/_random_layouts.py), runs the library
through its C ABI and the oracle on the same bytes, and compares every byte
of every output buffer and the error flag.  The trials are fixed by their
seeds, so a failure names a reproducible case; the CPU test
test_random_layouts_walk.py walks every one of them with an AddressSanitizer
build of the oracle over buffers of the device sizes first.
"""
import numpy as np
import pytest
import torch

import fp8_kv_quantization_amd as kv
from tests import _random_layouts as R
from tests._gpu import DEV, assert_cache_equal, check_flag, stream

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run_copy(L):
    dtype, off, T = L["dtype"], L["off"], L["T"]
    _say(f"copy row={L['row']} strides={L['k_stride']},{L['v_stride']} T={T} slots={L['slots']} "
         f"limit={L['limit']} vw={L['vw']} {dtype.__name__} istride={L['istride']} off={off}")
    kd = torch.zeros(L["k_in_bytes"], dtype=torch.uint8, device=DEV)
    vd = torch.zeros(L["v_in_bytes"], dtype=torch.uint8, device=DEV)
    kd[off:off + T * L["k_stride"]] = _dev(L["kb"].reshape(-1))
    vd[off:off + T * L["v_stride"]] = _dev(L["vb"].reshape(-1))
    kc = torch.full((L["cache_bytes"],), 0xFF, dtype=torch.uint8, device=DEV)
    vc = torch.full_like(kc, 0xFF)
    di = _dev(R.strided_indices(L["idx"], L["istride"]))
    st = kv.kvstore_copy(kd.data_ptr() + off, vd.data_ptr() + off, kc.data_ptr() + off,
                         vc.data_ptr() + off, di.data_ptr(),
                         kv.IDX_I64 if dtype == np.int64 else kv.IDX_I32, L["istride"], L["row"],
                         L["k_stride"], L["v_stride"], L["row"], T, L["limit"], stream())
    assert st == kv.OK
    return [kc, vc]


def run_fp8(L):
    op, H, D, P, T = L["op"], L["H"], L["D"], L["P"], L["T"]
    _say(f"{op} T={T} H={H} D={D} src={L['src']} P={P} pages={L['pages']} limit={L['limit']} "
         f"{L['dtype'].__name__} istride={L['istride']} in={L['k_in'][1] // 2},{L['v_in'][1] // 2} "
         f"kc={L['kcs']} vc={L['vcs']} ik={L['ik']} iv={L['iv']}")
    kd, vd = _dev(L["kb"]), _dev(L["vb"])
    kc = torch.full((L["kc_bytes"],), 0xFF, dtype=torch.uint8, device=DEV)
    vc = torch.full((L["vc_bytes"],), 0xFF, dtype=torch.uint8, device=DEV)
    di = _dev(R.strided_indices(L["idx"], L["istride"]))
    idt = kv.IDX_I64 if L["dtype"] == np.int64 else kv.IDX_I32
    sdt = kv.SRC_FP16 if L["src"] == "fp16" else kv.SRC_BF16
    if not L["dynamic"]:
        ik, iv = L["ik"], L["iv"]
        ikd = _dev(np.array([ik], dtype=np.uint32).view(np.float32)) if ik is not None else None
        ivd = _dev(np.array([iv], dtype=np.uint32).view(np.float32)) if iv is not None else None
        entry = kv.kvstore_fp8_paged_e5m2 if op == "e5m2" else kv.kvstore_fp8_paged
        st = entry(kd.data_ptr(), vd.data_ptr(), kc.data_ptr(), vc.data_ptr(), di.data_ptr(), idt,
                   L["istride"], sdt, H, D, *L["k_in"], *L["v_in"], *L["kcs"], *L["vcs"], T,
                   L["limit"], P, None if ikd is None else ikd.data_ptr(),
                   None if ivd is None else ivd.data_ptr(), stream())
        torch.cuda.synchronize()
        assert st == kv.OK
        return [kc, vc]
    ks = torch.full((L["ks_bytes"],), 0xFF, dtype=torch.uint8, device=DEV)
    vs = torch.full((L["vs_bytes"],), 0xFF, dtype=torch.uint8, device=DEV)
    st = kv.kvstore_fp8_paged_dynamic(
        kd.data_ptr(), vd.data_ptr(), kc.data_ptr(), vc.data_ptr(), di.data_ptr(), idt,
        L["istride"], sdt, H, D, *L["k_in"], *L["v_in"], *L["kcs"], *L["vcs"], ks.data_ptr(),
        vs.data_ptr(), kv.SCALE_PER_TOKEN_HEAD if L["per_head"] else kv.SCALE_PER_TOKEN,
        *L["kss"], *L["vss"], T, L["limit"], P, stream())
    torch.cuda.synchronize()
    assert st == kv.OK
    return [kc, vc, ks, vs]


@pytest.mark.parametrize("seed", R.SEEDS)
def test_random_layouts(seed):
    op, L = R.draw(seed)
    check_flag()
    got = run_copy(L) if op == "copy" else run_fp8(L)
    want, ost = R.run_oracle(op, L)
    _, first_bad, bad_count = ost
    st, fb, bc = check_flag()
    assert (fb, bc) == (first_bad, bad_count)
    assert st == (kv.ERR_OOB if bad_count else kv.OK)
    for i, (g, w) in enumerate(zip(got, want)):
        assert_cache_equal(g, w, f"buffer {i}")
