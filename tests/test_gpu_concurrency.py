"""GPU: store calls from several host threads, each on its own stream.

The library keeps no per-call host state beyond a per-device cache of one
device attribute, and the device flag is updated with atomics, so calls may
be issued concurrently.  Four threads (the binding releases the GIL) each
own a stream and their own caches and issue interleaved copy, FP8 and
dynamic-scale stores; afterwards every cache must match the oracle and the
shared flag must hold the smallest out-of-range token and the count over all
threads.
"""
import threading

import numpy as np
import pytest
import torch

import fp8_kv_quantization_amd as kv
import kvgen
import oracle
from tests._gpu import DEV, assert_cache_equal, check_flag, sentinel_cache, to_dev

pytestmark = pytest.mark.gpu

THREADS = 4
ROUNDS = 6


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


class Worker:
    """One thread's inputs, caches and expected results."""

    def __init__(self, n):
        self.copy = kvgen.workload(3, tokens=1500 + 37 * n, slots=1 << 13, seed=4000 + n)
        self.fp8 = kvgen.workload(4, tokens=700 + 11 * n, slots=64 * 32, seed=5000 + n)
        # one out-of-range index per worker in its copy batch, at token 100 + n
        self.bad_token = 100 + n
        self.copy.indices = self.copy.indices.copy()
        self.copy.indices[self.bad_token] = self.copy.slots + n
        c, f = self.copy, self.fp8
        self.k, self.v, self.idx = to_dev(c.k), to_dev(c.v), to_dev(c.indices)
        self.fk, self.fv, self.fidx = to_dev(f.k), to_dev(f.v), to_dev(f.indices)
        self.ik = to_dev(np.array([f.inv_k_bits], dtype=np.uint32).view(np.float32))
        self.iv = to_dev(np.array([f.inv_v_bits], dtype=np.uint32).view(np.float32))
        self.kc = sentinel_cache(c.slots, c.row_bytes)
        self.vc = sentinel_cache(c.slots, c.row_bytes)
        self.fkc = sentinel_cache(f.slots, f.row_elems)
        self.fvc = sentinel_cache(f.slots, f.row_elems)
        self.dkc = sentinel_cache(f.slots, f.row_elems)
        self.dvc = sentinel_cache(f.slots, f.row_elems)
        self.dks = sentinel_cache(f.slots, 4)
        self.dvs = sentinel_cache(f.slots, 4)
        self.stream = torch.cuda.Stream()
        self.status = []

    def run(self):
        c, f = self.copy, self.fp8
        H, D, P = f.num_heads, f.head_dim, f.page_size
        R = H * D
        ins = (f.in_stride_bytes, 2 * D)
        cs = (P * R, R, D)
        sh = self.stream.cuda_stream
        for _ in range(ROUNDS):
            self.status.append(kv.kvstore_copy(
                self.k.data_ptr(), self.v.data_ptr(), self.kc.data_ptr(), self.vc.data_ptr(),
                self.idx.data_ptr(), kv.IDX_I32, 1, c.row_bytes, c.in_stride_bytes,
                c.in_stride_bytes, c.row_bytes, c.num_tokens, c.slots, sh))
            self.status.append(kv.kvstore_fp8_paged(
                self.fk.data_ptr(), self.fv.data_ptr(), self.fkc.data_ptr(), self.fvc.data_ptr(),
                self.fidx.data_ptr(), kv.IDX_I32, 1, kv.SRC_BF16, H, D, *ins, *ins, *cs, *cs,
                f.num_tokens, f.slots, P, self.ik.data_ptr(), self.iv.data_ptr(), sh))
            self.status.append(kv.kvstore_fp8_paged_dynamic(
                self.fk.data_ptr(), self.fv.data_ptr(), self.dkc.data_ptr(), self.dvc.data_ptr(),
                self.fidx.data_ptr(), kv.IDX_I32, 1, kv.SRC_BF16, H, D, *ins, *ins, *cs, *cs,
                self.dks.data_ptr(), self.dvs.data_ptr(), kv.SCALE_PER_TOKEN, P * 4, 4, 0,
                P * 4, 4, 0, f.num_tokens, f.slots, P, sh))


def test_threads_on_separate_streams():
    _say(f"concurrency: {THREADS} threads x {ROUNDS} rounds x 3 stores")
    check_flag()
    workers = [Worker(n) for n in range(THREADS)]
    torch.cuda.synchronize()
    threads = [threading.Thread(target=w.run) for w in workers]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for w in workers:
        assert w.status == [kv.OK] * (3 * ROUNDS)
    # each copy call skips its worker's one bad token: ROUNDS reports per worker
    assert check_flag() == (kv.ERR_OOB, min(w.bad_token for w in workers), THREADS * ROUNDS)
    for n, w in enumerate(workers):
        okc, ovc, st = oracle.run_case(w.copy)
        assert st[1:] == (w.bad_token, 1)
        assert_cache_equal(w.kc, okc, f"worker {n} copy k_cache")
        assert_cache_equal(w.vc, ovc, f"worker {n} copy v_cache")
        ofk, ofv, _ = oracle.run_case(w.fp8)
        assert_cache_equal(w.fkc, ofk, f"worker {n} fp8 k_cache")
        assert_cache_equal(w.fvc, ofv, f"worker {n} fp8 v_cache")
        odk, odv, odks, odvs, _ = oracle.run_case_dynamic(w.fp8, per_head=False)
        assert_cache_equal(w.dkc, odk, f"worker {n} dynamic k_cache")
        assert_cache_equal(w.dvc, odv, f"worker {n} dynamic v_cache")
        assert_cache_equal(w.dks, odks.view(np.uint8), f"worker {n} dynamic k_scales")
        assert_cache_equal(w.dvs, odvs.view(np.uint8), f"worker {n} dynamic v_scales")
