"""GPU: batches above 2^24 tokens, which the library runs as several launches.

Every entry point stores 2^24 + 4099 tokens: one full run of 2^24 tokens and a
ragged second run.  Tokens 2^24 - 1, 2^24 and the last carry out-of-range
indices, so the error flag must name the smallest of them and count all three
across both launches.

Copy: every other token's row must sit at its slot (byte identity, the
definition of the copy) and every slot that no token names must keep the 0xFF
sentinel.  FP8 stores: the input rows repeat with a period of 4096 tokens, the
oracle stores one period (4096 tokens), and every stored row (and scale) of
the whole batch must equal the oracle's row for its position in the period.
"""
import numpy as np
import pytest
import torch

import fp8_kv_quantization_amd as kv
import kvgen
import oracle
from tests._gpu import DEV, check_flag, stream

pytestmark = pytest.mark.gpu

BATCH = (1 << 24) + 4099
PERIOD = 4096
BAD = [(1 << 24) - 1, 1 << 24, BATCH - 1]
CHUNK = 1 << 22


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _clean_flag():
    check_flag()
    yield
    torch.cuda.synchronize()


def _indices(slots, seed):
    """int32 slots of a seeded permutation, with the BAD tokens out of range.
    Returns (host int32 indices, device int64 slots of the valid tokens,
    device bool mask of the valid tokens)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    idx = torch.randperm(slots, generator=g)[:BATCH].to(torch.int32)
    idx[BAD] = slots
    good = torch.ones(BATCH, dtype=torch.bool)
    good[BAD] = False
    return idx, idx.to(DEV), good.to(DEV)


def _untouched_keep_sentinel(cache, idx_dev, good_dev):
    written = torch.zeros(cache.shape[0], dtype=torch.bool, device=DEV)
    written[idx_dev[good_dev].long()] = True
    assert bool((cache[~written] == 0xFF).all())


def _rows_match(cache, idx_dev, good_dev, want_row):
    """cache[idx[t]] == want_row(t0, t1)[t - t0] for every valid token t."""
    for s in range(0, BATCH, CHUNK):
        e = min(BATCH, s + CHUNK)
        sel = good_dev[s:e]
        got = cache[idx_dev[s:e].long()[sel]]
        want = want_row(s, e)[sel]
        assert torch.equal(got, want), f"rows of tokens [{s}, {e}) differ"


@pytest.mark.parametrize("row", [132, 16])
def test_copy_max_batch(row):
    # 132-byte rows (33 four-byte lanes) take one wave per row; 16-byte rows
    # are packed 128 to a wave.
    _say(f"copy max batch T={BATCH} row={row}")
    slots = BATCH + 8192
    idx, idx_dev, good_dev = _indices(slots, row)
    g = torch.Generator(device=DEV).manual_seed(row)
    k = torch.randint(0, 256, (BATCH, row), dtype=torch.uint8, device=DEV, generator=g)
    v = torch.randint(0, 256, (BATCH, row), dtype=torch.uint8, device=DEV, generator=g)
    kc = torch.full((slots, row), 0xFF, dtype=torch.uint8, device=DEV)
    vc = torch.full_like(kc, 0xFF)
    st = kv.kvstore_copy(k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                         idx_dev.data_ptr(), kv.IDX_I32, 1, row, row, row, row, BATCH, slots,
                         stream())
    assert st == kv.OK
    assert check_flag() == (kv.ERR_OOB, BAD[0], len(BAD))
    _rows_match(kc, idx_dev, good_dev, lambda s, e: k[s:e])
    _rows_match(vc, idx_dev, good_dev, lambda s, e: v[s:e])
    _untouched_keep_sentinel(kc, idx_dev, good_dev)
    _untouched_keep_sentinel(vc, idx_dev, good_dev)


def _period_inputs(H, D, seed):
    """bf16 bits [PERIOD, H*D] for K and V: normal values at mixed magnitudes
    with a few raw 16-bit patterns (NaN, inf, subnormals)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((2, PERIOD, H * D)).astype(np.float32)
    x *= np.float32(300.0) ** rng.random((2, PERIOD, 1)).astype(np.float32)
    bits = kvgen._round_f32_to_bf16_bits(x)
    raw = rng.random(bits.shape) < 0.002
    bits = np.where(raw, rng.integers(0, 65536, bits.shape), bits).astype(np.uint16)
    return bits[0], bits[1]


def _repeat(bits):
    reps = -(-BATCH // PERIOD)
    d = torch.from_numpy(bits.view(np.int16)).to(DEV)
    return d.repeat(reps, 1)[:BATCH].contiguous()


def _periodic(ref_rows):
    """want_row for rows that repeat with the period."""
    ref = torch.from_numpy(np.ascontiguousarray(ref_rows)).to(DEV)

    def want(s, e):
        return ref[torch.arange(s, e, device=DEV) % PERIOD]
    return want


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
def test_fp8_max_batch(fmt):
    H, D, P = 1, 16, 64
    _say(f"fp8 {fmt} max batch T={BATCH} H={H} D={D}")
    slots = -(-(BATCH + 8192) // P) * P
    idx, idx_dev, good_dev = _indices(slots, 17)
    kb, vb = _period_inputs(H, D, 17)
    k, v = _repeat(kb), _repeat(vb)
    ik = torch.tensor([0.4], dtype=torch.float32, device=DEV)
    iv = torch.tensor([1 / 1.7], dtype=torch.float32, device=DEV)
    kc = torch.full((slots, H * D), 0xFF, dtype=torch.uint8, device=DEV)
    vc = torch.full_like(kc, 0xFF)
    entry = kv.kvstore_fp8_paged_e5m2 if fmt == "e5m2" else kv.kvstore_fp8_paged
    ins = (2 * H * D, 2 * D)
    cs = (P * H * D, H * D, D)
    st = entry(k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(), idx_dev.data_ptr(),
               kv.IDX_I32, 1, kv.SRC_BF16, H, D, *ins, *ins, *cs, *cs, BATCH, slots, P,
               ik.data_ptr(), iv.data_ptr(), stream())
    assert st == kv.OK
    assert check_flag() == (kv.ERR_OOB, BAD[0], len(BAD))
    # the oracle on one period, token j at slot j
    okc = np.full((PERIOD, H * D), 0xFF, dtype=np.uint8)
    ovc = np.full_like(okc, 0xFF)
    bits = lambda t: int(t.cpu().view(torch.int32).item())
    ost = oracle.fp8_paged(kb, vb, okc, ovc, np.arange(PERIOD, dtype=np.int32), src_dtype="bf16",
                           num_heads=H, head_dim=D, k_strides=ins, v_strides=ins, kc_strides=cs,
                           vc_strides=cs, size_limit=PERIOD, page_size=P, inv_k_bits=bits(ik),
                           inv_v_bits=bits(iv), fmt=fmt)
    assert ost == (PERIOD, -1, 0)
    _rows_match(kc, idx_dev, good_dev, _periodic(okc))
    _rows_match(vc, idx_dev, good_dev, _periodic(ovc))
    _untouched_keep_sentinel(kc, idx_dev, good_dev)
    _untouched_keep_sentinel(vc, idx_dev, good_dev)


@pytest.mark.parametrize("per_head", [False, True])
def test_fp8_dynamic_max_batch(per_head):
    H, D, P = 2, 16, 64
    G = H if per_head else 1
    _say(f"fp8 dynamic per_head={per_head} max batch T={BATCH} H={H} D={D}")
    slots = -(-(BATCH + 8192) // P) * P
    idx, idx_dev, good_dev = _indices(slots, 29)
    kb, vb = _period_inputs(H, D, 29)
    k, v = _repeat(kb), _repeat(vb)
    kc = torch.full((slots, H * D), 0xFF, dtype=torch.uint8, device=DEV)
    vc = torch.full_like(kc, 0xFF)
    ks = torch.full((slots, 4 * G), 0xFF, dtype=torch.uint8, device=DEV)
    vs = torch.full_like(ks, 0xFF)
    ins = (2 * H * D, 2 * D)
    cs = (P * H * D, H * D, D)
    ss = (P * G * 4, G * 4, 4)
    st = kv.kvstore_fp8_paged_dynamic(
        k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(), idx_dev.data_ptr(), kv.IDX_I32,
        1, kv.SRC_BF16, H, D, *ins, *ins, *cs, *cs, ks.data_ptr(), vs.data_ptr(),
        kv.SCALE_PER_TOKEN_HEAD if per_head else kv.SCALE_PER_TOKEN, *ss, *ss, BATCH, slots, P,
        stream())
    assert st == kv.OK
    assert check_flag() == (kv.ERR_OOB, BAD[0], len(BAD))
    okc = np.full((PERIOD, H * D), 0xFF, dtype=np.uint8)
    ovc = np.full_like(okc, 0xFF)
    oks = np.full((PERIOD, G), 0xFFFFFFFF, dtype=np.uint32)
    ovs = np.full_like(oks, 0xFFFFFFFF)
    ost = oracle.fp8_paged_dynamic(kb, vb, okc, ovc, np.arange(PERIOD, dtype=np.int32), oks, ovs,
                                   src_dtype="bf16", num_heads=H, head_dim=D, k_strides=ins,
                                   v_strides=ins, kc_strides=cs, vc_strides=cs, ks_strides=ss,
                                   vs_strides=ss, per_head=per_head, size_limit=PERIOD,
                                   page_size=P)
    assert ost == (PERIOD, -1, 0)
    _rows_match(kc, idx_dev, good_dev, _periodic(okc))
    _rows_match(vc, idx_dev, good_dev, _periodic(ovc))
    _rows_match(ks, idx_dev, good_dev, _periodic(oks.view(np.uint8)))
    _rows_match(vs, idx_dev, good_dev, _periodic(ovs.view(np.uint8)))
    _untouched_keep_sentinel(kc, idx_dev, good_dev)
    _untouched_keep_sentinel(ks, idx_dev, good_dev)
