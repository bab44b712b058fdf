"""GPU: store calls recorded once into a HIP graph and replayed.

A store call launches kernels on the caller's stream and nothing else: no
allocation, no copy, no memset, no host synchronisation.  The index array and
the inverse scales are read through device pointers when the kernel runs, which
is why the fused FP8 path of sglang "trtllm_fp8_kv_kernel.py" (the
set_kv_buffer wrapper) takes its scales as device values: a captured call then
follows whatever those buffers hold at replay time.

Each test captures calls once and replays the graph three times.  Between
replays, eager work on the same stream overwrites the inputs, indices and
scales with a new seeded case and resets the caches to the 0xFF sentinel; after
each replay every byte of every output buffer is compared with the oracle run
on that case, and the error flag with the oracle's count.  The last two tests
cover kvstore_take_error, the error read that can sit inside a graph.
"""
import dataclasses

import numpy as np
import pytest
import torch

import fp8_kv_quantization_amd as kv
import kvgen
import oracle
from tests._gpu import DEV, assert_cache_equal, check_flag, sentinel_cache, stream, to_dev

pytestmark = pytest.mark.gpu

SCALE_BITS = [(0x3ECCCCCD, 0x3F169696), (0x41200000, 0x3A83126F), (0x3F800000, 0x3ECCCCCD)]


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _clean_flag():
    check_flag()
    yield
    torch.cuda.synchronize()


def _capture(calls):
    """Run ``calls`` once eagerly on a side stream, then record them into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for call in calls:
            assert call() == kv.OK
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    check_flag()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for call in calls:
            assert call() == kv.OK
    torch.cuda.synchronize()
    return g


def _replay(g):
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()


def _f32(bits):
    return to_dev(np.array([bits], dtype=np.uint32).view(np.float32))


def _expect_flag(st):
    _, first_bad, count = st
    assert check_flag() == ((kv.ERR_OOB, first_bad, count) if count else (kv.OK, -1, 0))


def _with_bad_index(c, t):
    c.indices = c.indices.copy()
    c.indices[t] = c.slots
    return c


@pytest.mark.parametrize("n,tokens,slots", [(1, 3000, 1 << 13), (3, 3000, 1 << 14),
                                            (5, 2000, 1 << 13)])
def test_graph_copy(n, tokens, slots):
    cases = [kvgen.workload(n, tokens=tokens, slots=slots, seed=500 + i) for i in range(3)]
    _with_bad_index(cases[1], 17)
    c0 = cases[0]
    k, v, idx = to_dev(c0.k), to_dev(c0.v), to_dev(c0.indices)
    kc = sentinel_cache(c0.slots, c0.row_bytes)
    vc = sentinel_cache(c0.slots, c0.row_bytes)
    code = kv.IDX_I64 if c0.indices.dtype == np.int64 else kv.IDX_I32

    def call():
        return kv.kvstore_copy(k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                               idx.data_ptr(), code, 1, c0.row_bytes, c0.in_stride_bytes,
                               c0.in_stride_bytes, c0.row_bytes, c0.num_tokens, c0.slots,
                               stream())

    g = _capture([call])
    for i, c in enumerate(cases):
        _say(f"graph copy {c.name} replay {i} T={c.num_tokens} row={c.row_bytes}")
        k.copy_(to_dev(c.k))
        v.copy_(to_dev(c.v))
        idx.copy_(to_dev(c.indices))
        kc.fill_(0xFF)
        vc.fill_(0xFF)
        _replay(g)
        okc, ovc, st = oracle.run_case(c)
        _expect_flag(st)
        assert_cache_equal(kc, okc, f"k_cache replay {i}")
        assert_cache_equal(vc, ovc, f"v_cache replay {i}")


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
def test_graph_fp8_scales_follow_device_values(fmt):
    cases = [kvgen.workload(4, tokens=2000, slots=64 * 64, seed=600 + i) for i in range(3)]
    cases = [dataclasses.replace(c, inv_k_bits=sk, inv_v_bits=sv)
             for c, (sk, sv) in zip(cases, SCALE_BITS)]
    _with_bad_index(cases[2], 1999)
    c0 = cases[0]
    H, D, P = c0.num_heads, c0.head_dim, c0.page_size
    row = H * D
    k, v, idx = to_dev(c0.k), to_dev(c0.v), to_dev(c0.indices)
    ik, iv = _f32(c0.inv_k_bits), _f32(c0.inv_v_bits)
    kc = sentinel_cache(c0.slots, row)
    vc = sentinel_cache(c0.slots, row)
    entry = kv.kvstore_fp8_paged_e5m2 if fmt == "e5m2" else kv.kvstore_fp8_paged
    ins = (c0.in_stride_bytes, 2 * D)
    cs = (P * row, row, D)

    def call():
        return entry(k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(), idx.data_ptr(),
                     kv.IDX_I32, 1, kv.SRC_BF16, H, D, *ins, *ins, *cs, *cs, c0.num_tokens,
                     c0.slots, P, ik.data_ptr(), iv.data_ptr(), stream())

    g = _capture([call])
    for i, c in enumerate(cases):
        _say(f"graph fp8 {fmt} replay {i} T={c.num_tokens} inv=({c.inv_k_bits:#x}, "
             f"{c.inv_v_bits:#x})")
        k.copy_(to_dev(c.k))
        v.copy_(to_dev(c.v))
        idx.copy_(to_dev(c.indices))
        ik.copy_(_f32(c.inv_k_bits))
        iv.copy_(_f32(c.inv_v_bits))
        kc.fill_(0xFF)
        vc.fill_(0xFF)
        _replay(g)
        okc, ovc, st = oracle.run_case(c, fmt=fmt)
        _expect_flag(st)
        assert_cache_equal(kc, okc, f"k_cache replay {i}")
        assert_cache_equal(vc, ovc, f"v_cache replay {i}")


@pytest.mark.parametrize("per_head", [False, True])
def test_graph_fp8_dynamic(per_head):
    cases = [kvgen.workload(4, tokens=1500, slots=64 * 48, seed=700 + i) for i in range(3)]
    _with_bad_index(cases[1], 0)
    c0 = cases[0]
    H, D, P = c0.num_heads, c0.head_dim, c0.page_size
    G = H if per_head else 1
    row = H * D
    k, v, idx = to_dev(c0.k), to_dev(c0.v), to_dev(c0.indices)
    kc = sentinel_cache(c0.slots, row)
    vc = sentinel_cache(c0.slots, row)
    ks = sentinel_cache(c0.slots, 4 * G)
    vs = sentinel_cache(c0.slots, 4 * G)
    ins = (c0.in_stride_bytes, 2 * D)
    cs = (P * row, row, D)
    ss = (P * G * 4, G * 4, 4 if per_head else 0)
    gran = kv.SCALE_PER_TOKEN_HEAD if per_head else kv.SCALE_PER_TOKEN

    def call():
        return kv.kvstore_fp8_paged_dynamic(
            k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(), idx.data_ptr(), kv.IDX_I32,
            1, kv.SRC_BF16, H, D, *ins, *ins, *cs, *cs, ks.data_ptr(), vs.data_ptr(), gran, *ss,
            *ss, c0.num_tokens, c0.slots, P, stream())

    g = _capture([call])
    for i, c in enumerate(cases):
        _say(f"graph fp8 dynamic per_head={per_head} replay {i} T={c.num_tokens}")
        k.copy_(to_dev(c.k))
        v.copy_(to_dev(c.v))
        idx.copy_(to_dev(c.indices))
        for buf in (kc, vc, ks, vs):
            buf.fill_(0xFF)
        _replay(g)
        okc, ovc, oks, ovs, st = oracle.run_case_dynamic(c, per_head)
        _expect_flag(st)
        assert_cache_equal(kc, okc, f"k_cache replay {i}")
        assert_cache_equal(vc, ovc, f"v_cache replay {i}")
        assert_cache_equal(ks, oks.view(np.uint8), f"k_scales replay {i}")
        assert_cache_equal(vs, ovs.view(np.uint8), f"v_scales replay {i}")


def test_graph_step_copy_then_fp8():
    """One graph holding a copy and an FP8 store, as one step of a serving loop."""
    cc = [kvgen.workload(3, tokens=2048, slots=1 << 13, seed=800 + i) for i in range(3)]
    fc = [kvgen.workload(4, tokens=1024, slots=64 * 32, seed=900 + i) for i in range(3)]
    c0, f0 = cc[0], fc[0]
    H, D, P = f0.num_heads, f0.head_dim, f0.page_size
    row = H * D
    k, v, idx = to_dev(c0.k), to_dev(c0.v), to_dev(c0.indices)
    fk, fv, fidx = to_dev(f0.k), to_dev(f0.v), to_dev(f0.indices)
    ik, iv = _f32(f0.inv_k_bits), _f32(f0.inv_v_bits)
    kc = sentinel_cache(c0.slots, c0.row_bytes)
    vc = sentinel_cache(c0.slots, c0.row_bytes)
    fkc = sentinel_cache(f0.slots, row)
    fvc = sentinel_cache(f0.slots, row)
    ins = (f0.in_stride_bytes, 2 * D)
    cs = (P * row, row, D)

    def copy_call():
        return kv.kvstore_copy(k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                               idx.data_ptr(), kv.IDX_I32, 1, c0.row_bytes, c0.in_stride_bytes,
                               c0.in_stride_bytes, c0.row_bytes, c0.num_tokens, c0.slots,
                               stream())

    def fp8_call():
        return kv.kvstore_fp8_paged(fk.data_ptr(), fv.data_ptr(), fkc.data_ptr(), fvc.data_ptr(),
                                    fidx.data_ptr(), kv.IDX_I32, 1, kv.SRC_BF16, H, D, *ins, *ins,
                                    *cs, *cs, f0.num_tokens, f0.slots, P, ik.data_ptr(),
                                    iv.data_ptr(), stream())

    g = _capture([copy_call, fp8_call])
    for i, (c, f) in enumerate(zip(cc, fc)):
        _say(f"graph step replay {i}")
        k.copy_(to_dev(c.k))
        v.copy_(to_dev(c.v))
        idx.copy_(to_dev(c.indices))
        fk.copy_(to_dev(f.k))
        fv.copy_(to_dev(f.v))
        fidx.copy_(to_dev(f.indices))
        for buf in (kc, vc, fkc, fvc):
            buf.fill_(0xFF)
        _replay(g)
        assert check_flag() == (kv.OK, -1, 0)
        okc, ovc, _ = oracle.run_case(c)
        ofk, ofv, _ = oracle.run_case(f)
        assert_cache_equal(kc, okc, f"copy k_cache replay {i}")
        assert_cache_equal(vc, ovc, f"copy v_cache replay {i}")
        assert_cache_equal(fkc, ofk, f"fp8 k_cache replay {i}")
        assert_cache_equal(fvc, ofv, f"fp8 v_cache replay {i}")


def test_take_error_eager_collects_and_clears():
    """kvstore_take_error after two stores with bad tokens: the smallest bad
    token and the total count land in the device buffer, and the flag is
    cleared (a later check finds nothing)."""
    c = kvgen.workload(1, tokens=200, slots=1024)
    c.indices = c.indices.copy()
    c.indices[[9, 150]] = c.slots
    c2 = kvgen.workload(1, tokens=200, slots=1024, seed=77)
    c2.indices = c2.indices.copy()
    c2.indices[4] = -1
    kc = sentinel_cache(c.slots, c.row_bytes)
    vc = sentinel_cache(c.slots, c.row_bytes)
    out = torch.full((2,), 12345, dtype=torch.int64, device=DEV)
    for case in (c, c2):
        k, v, idx = to_dev(case.k), to_dev(case.v), to_dev(case.indices)
        assert kv.kvstore_copy(k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                               idx.data_ptr(), kv.IDX_I32, 1, case.row_bytes, case.in_stride_bytes,
                               case.in_stride_bytes, case.row_bytes, case.num_tokens, case.slots,
                               stream()) == kv.OK
    kv.take_error(out)
    torch.cuda.synchronize()
    assert out.tolist() == [4, 3]
    assert check_flag() == (kv.OK, -1, 0)
    kv.take_error(out)                      # nothing since: -1, 0
    torch.cuda.synchronize()
    assert out.tolist() == [-1, 0]


def test_take_error_inside_a_graph():
    """A graph holding a store and the error take: each replay reports the
    bad tokens of that replay only, with no host synchronisation in the graph."""
    c = kvgen.workload(3, tokens=1000, slots=1 << 13, seed=31)
    k, v, idx = to_dev(c.k), to_dev(c.v), to_dev(c.indices)
    good = idx.clone()
    kc = sentinel_cache(c.slots, c.row_bytes)
    vc = sentinel_cache(c.slots, c.row_bytes)
    out = torch.zeros(2, dtype=torch.int64, device=DEV)

    def store():
        return kv.kvstore_copy(k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                               idx.data_ptr(), kv.IDX_I32, 1, c.row_bytes, c.in_stride_bytes,
                               c.in_stride_bytes, c.row_bytes, c.num_tokens, c.slots, stream())

    def take():
        return kv.kvstore_take_error(out.data_ptr(), stream())

    g = _capture([store, take])
    for i, bad in enumerate(([], [333], [], [12, 999, 500])):
        _say(f"graph take_error replay {i} bad={bad}")
        idx.copy_(good)
        for t in bad:
            idx[t] = c.slots + t
        out.fill_(12345)
        _replay(g)
        assert out.tolist() == ([min(bad), len(bad)] if bad else [-1, 0])
        assert check_flag() == (kv.OK, -1, 0)
