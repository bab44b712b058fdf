"""The per-device error flag under contention: a batch whose tokens are
nearly all out of range makes every rejected token race one compare-and-swap
on the same 64-bit word (several per wave in the packed small-row kernel).
The flag must then hold exactly the count and the smallest rejected token,
the in-range rows must be written as the oracle writes them, and nothing else
may change."""
import numpy as np
import pytest
import torch

import fp8_kv_quantization_amd as kv
import kvgen
import oracle
from tests._gpu import assert_cache_equal, check_flag, run_copy, run_fp8, sentinel_cache, to_dev

pytestmark = pytest.mark.gpu

T = 1 << 16                 # tokens per call
SLOTS = 4096                # cache slots; every index >= SLOTS is rejected
GOOD = {0: 7, 2: 4095, 3000: 0, 65535: 1234}   # the only in-range tokens


def _indices(dt):
    idx = (SLOTS + np.arange(T, dtype=np.int64)).astype(dt)
    for t, slot in GOOD.items():
        idx[t] = slot
    return idx


@pytest.fixture(autouse=True)
def _clean_flag():
    st, _, _ = check_flag()
    assert st in (kv.OK, kv.ERR_OOB)
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("row_elems,i64", [(1024, False), (128, True), (20, False)],
                         ids=["2KiB_rows", "256B_rows_packed", "40B_rows_packed"])
def test_copy_flag_counts_every_racing_report(row_elems, i64):
    c = kvgen.workload(2, tokens=T, slots=T)
    c.slots = SLOTS
    c.k = np.ascontiguousarray(c.k[:, :row_elems])
    c.v = np.ascontiguousarray(c.v[:, :row_elems])
    c.num_heads, c.head_dim, c.in_stride_elems = 1, row_elems, row_elems
    c.indices = _indices(np.int64 if i64 else np.int32)
    c.idx_dtype = kvgen.I64 if i64 else kvgen.I32
    print(f"[gpu-case] flag contention copy row={2 * row_elems} B i64={i64}", flush=True)
    kc = sentinel_cache(SLOTS, c.row_bytes)
    vc = sentinel_cache(SLOTS, c.row_bytes)
    assert run_copy(c, kc, vc) == kv.OK
    n_bad = T - len(GOOD)
    assert check_flag() == (kv.ERR_OOB, 1, n_bad)
    assert check_flag() == (kv.OK, -1, 0)
    okc, ovc, ost = oracle.run_case(c)
    assert ost == (len(GOOD), 1, n_bad)
    assert_cache_equal(kc, okc, "k_cache")
    assert_cache_equal(vc, ovc, "v_cache")


def test_fp8_flag_counts_every_racing_report():
    c = kvgen.workload(4, tokens=T, slots=T)
    c.slots = SLOTS
    c.indices = _indices(np.int32)
    print("[gpu-case] flag contention fp8", flush=True)
    kc = sentinel_cache(SLOTS, c.row_elems)
    vc = sentinel_cache(SLOTS, c.row_elems)
    assert run_fp8(c, kc, vc) == kv.OK
    n_bad = T - len(GOOD)
    assert check_flag() == (kv.ERR_OOB, 1, n_bad)
    okc, ovc, ost = oracle.run_case(c)
    assert ost == (len(GOOD), 1, n_bad)
    assert_cache_equal(kc, okc, "k_cache")
    assert_cache_equal(vc, ovc, "v_cache")


@pytest.mark.parametrize("per_head", [False, True])
def test_dynamic_flag_counts_every_racing_report_and_take_clears(per_head):
    c = kvgen.workload(4, tokens=T, slots=T)
    c.slots = SLOTS
    c.indices = _indices(np.int32)
    H, D, P = c.num_heads, c.head_dim, c.page_size
    G = H if per_head else 1
    row = c.row_elems
    print(f"[gpu-case] flag contention dynamic per_head={per_head}", flush=True)
    kc = sentinel_cache(SLOTS, row)
    vc = sentinel_cache(SLOTS, row)
    ks = torch.full((SLOTS, G), -1, dtype=torch.int32, device="cuda:0").view(torch.float32)
    vs = torch.full((SLOTS, G), -1, dtype=torch.int32, device="cuda:0").view(torch.float32)
    k, v, idx = to_dev(c.k), to_dev(c.v), to_dev(c.indices)
    sh = torch.cuda.current_stream().cuda_stream
    st = kv.kvstore_fp8_paged_dynamic(
        k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(), idx.data_ptr(), kv.IDX_I32, 1,
        kv.SRC_BF16, H, D, c.in_stride_bytes, 2 * D, c.in_stride_bytes, 2 * D, P * row, row, D,
        P * row, row, D, ks.data_ptr(), vs.data_ptr(),
        kv.SCALE_PER_TOKEN_HEAD if per_head else kv.SCALE_PER_TOKEN,
        P * G * 4, G * 4, 4, P * G * 4, G * 4, 4, T, SLOTS, P, sh)
    assert st == kv.OK
    # the graph-capturable take: same word, taken on the stream, no sync
    out = torch.full((2,), 7, dtype=torch.int64, device="cuda:0")
    kv.take_error(out)
    torch.cuda.synchronize()
    n_bad = T - len(GOOD)
    assert out.tolist() == [1, n_bad]
    assert check_flag() == (kv.OK, -1, 0)
    okc, ovc, oks, ovs, ost = oracle.run_case_dynamic(c, per_head)
    assert ost == (len(GOOD), 1, n_bad)
    assert_cache_equal(kc, okc, "k_cache")
    assert_cache_equal(vc, ovc, "v_cache")
    np.testing.assert_array_equal(ks.view(torch.int32).cpu().numpy().view(np.uint32), oks)
    np.testing.assert_array_equal(vs.view(torch.int32).cpu().numpy().view(np.uint32), ovs)
