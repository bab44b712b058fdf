"""GPU parity of the dynamic-scale FP8 paged store against the CPU oracle.

Every byte of both FP8 caches and both fp32 scale caches (all sentinel-filled)
is compared with the oracle's, for per-token and per-token-head scales, bf16
and fp16 sources, the FP8 workload's shape at reduced and full size, head
shapes from 1x16 up to the 4096-element limit, edge groups (zeros, NaN,
infinities, tiny values), padded layouts with a divide-path page size, and
out-of-range indices.
"""
import numpy as np
import pytest
import torch

import fp8_kv_quantization_amd as kv
import kvgen
import oracle
from tests._gpu import DEV, assert_cache_equal, check_flag, sentinel_cache, stream, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _clean_flag():
    check_flag()
    yield
    torch.cuda.synchronize()


def run_dynamic(c, per_head, kc, vc, ks, vs, kc_strides=None, sc_strides=None, in_strides=None,
                k_dev=None, v_dev=None, size_limit=None):
    H, D, P = c.num_heads, c.head_dim, c.page_size
    row = H * D
    G = H if per_head else 1
    k = to_dev(c.k) if k_dev is None else k_dev
    v = to_dev(c.v) if v_dev is None else v_dev
    idx = to_dev(c.indices)
    ins = in_strides or (c.in_stride_bytes, 2 * D)
    kcs = kc_strides or (P * row, row, D)
    scs = sc_strides or (P * G * 4, G * 4, 4 if per_head else 0)
    st = kv.kvstore_fp8_paged_dynamic(
        k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(), idx.data_ptr(),
        kv.IDX_I64 if c.indices.dtype == np.int64 else kv.IDX_I32, 1,
        kv.SRC_FP16 if c.src_dtype == "fp16" else kv.SRC_BF16, H, D, ins[0], ins[1], ins[0],
        ins[1], kcs[0], kcs[1], kcs[2], kcs[0], kcs[1], kcs[2], ks.data_ptr(), vs.data_ptr(),
        kv.SCALE_PER_TOKEN_HEAD if per_head else kv.SCALE_PER_TOKEN, scs[0], scs[1], scs[2],
        scs[0], scs[1], scs[2], c.num_tokens, c.slots if size_limit is None else size_limit, P,
        stream())
    torch.cuda.synchronize()
    return st


def parity(c, per_head):
    _say(f"dynamic per_head={per_head} {c.name} T={c.num_tokens} H={c.num_heads} D={c.head_dim} "
         f"{c.src_dtype}")
    G = c.num_heads if per_head else 1
    kc = sentinel_cache(c.slots, c.row_elems)
    vc = sentinel_cache(c.slots, c.row_elems)
    ks = sentinel_cache(c.slots, 4 * G)
    vs = sentinel_cache(c.slots, 4 * G)
    assert run_dynamic(c, per_head, kc, vc, ks, vs) == kv.OK
    assert check_flag() == (kv.OK, -1, 0)
    okc, ovc, oks, ovs, st = oracle.run_case_dynamic(c, per_head)
    assert st == (c.num_tokens, -1, 0)
    assert_cache_equal(kc, okc, "k_cache")
    assert_cache_equal(vc, ovc, "v_cache")
    assert_cache_equal(ks, oks.view(np.uint8), "k_scales")
    assert_cache_equal(vs, ovs.view(np.uint8), "v_scales")


def fp8_case(tokens=300, pages=16, src="bf16", i64=False):
    c = kvgen.workload(4, tokens=tokens, slots=pages * 64)
    c.src_dtype = src
    if i64:
        c.indices = c.indices.astype(np.int64)
        c.idx_dtype = "i64"
    return c


@pytest.mark.parametrize("per_head", [False, True])
@pytest.mark.parametrize("src,i64", [("bf16", False), ("fp16", True)])
def test_dynamic_reduced(per_head, src, i64):
    parity(fp8_case(src=src, i64=i64), per_head)


@pytest.mark.parametrize("per_head", [False, True])
def test_dynamic_full_size(per_head):
    parity(kvgen.workload(4), per_head)


@pytest.mark.parametrize("heads,dim,modes", [(1, 16, (False, True)), (3, 48, (False,)),
                                             (8, 64, (False, True)), (16, 128, (False, True)),
                                             (32, 128, (False, True)), (2, 576, (False,)),
                                             (4, 1024, (False, True)), (2, 32, (True,)),
                                             (4, 256, (False, True)), (8, 512, (False, True)),
                                             (256, 16, (False, True)), (128, 32, (True,))])
@pytest.mark.parametrize("src", ["bf16", "fp16"])
def test_dynamic_head_shapes(heads, dim, modes, src):
    # Rows of one to four passes, some ending inside a pass (2 x 576), in
    # both source formats (fp16 rows of several passes load every group,
    # clamped to the row, and zero those past it); 256 heads of 16 is the
    # most head scales a row can have (every lane group a head).
    rng = np.random.Generator(np.random.PCG64(heads * 7 + dim))
    T, P, pages = 150, 16, 12
    x = rng.standard_normal((2, T, heads * dim), dtype=np.float32)
    x *= np.exp(rng.standard_normal((2, T, heads, 1), dtype=np.float32) * 3).repeat(dim, 3).reshape(x.shape)
    if src == "bf16":
        bits = kvgen._round_f32_to_bf16_bits(x)
    else:
        bits = np.clip(x, -60000, 60000).astype(np.float16).view(np.uint16)
    idx = rng.permutation(P * pages)[:T].astype(np.int32)
    c = kvgen.Case(name=f"h{heads}d{dim}", kind="fp8", src_dtype=src, num_tokens=T,
                   num_heads=heads, head_dim=dim, in_stride_elems=heads * dim, k=bits[0],
                   v=bits[1], indices=idx, idx_dtype="i32", slots=P * pages, page_size=P)
    for per_head in modes:
        parity(c, per_head)


@pytest.mark.parametrize("per_head", [False, True])
def test_dynamic_edge_groups(per_head):
    c = fp8_case(tokens=40, pages=1)
    f = lambda val: kvgen._round_f32_to_bf16_bits(np.full(1024, val, dtype=np.float32))
    c.k[0, :] = 0                   # zeros
    c.k[1, 5] = 0x7FC1              # a NaN
    c.k[1, 700] = 0xFF81            # a negative NaN in another head
    c.k[2, 7] = 0xFF80              # -inf
    c.k[3, :] = f(1e-39)            # tiny
    c.k[4, :] = 0x8000              # -0 only
    c.k[5, 130:140] = 0x7F80        # +inf in head 1
    c.v[6, :] = f(3e38)             # huge (bf16 rounds to inf? no: finite)
    parity(c, per_head)


@pytest.mark.parametrize("per_head", [False, True])
def test_dynamic_padded_layouts(per_head):
    c = fp8_case(tokens=250, pages=8)
    P = 48
    c.page_size = P
    c.slots = (c.slots // P) * P
    keep = c.indices < c.slots
    c.indices, c.k, c.v = c.indices[keep].copy(), c.k[keep].copy(), c.v[keep].copy()
    c.num_tokens = int(keep.sum())
    H, D, T = c.num_heads, c.head_dim, c.num_tokens
    sh_in = D + 8
    bk = np.full((T, H, sh_in), kvgen.PAD_POISON, dtype=np.uint16)
    bv = np.full_like(bk, kvgen.PAD_POISON)
    bk[:, :, :D] = c.k.reshape(T, H, D)
    bv[:, :, :D] = c.v.reshape(T, H, D)
    sh, so = D + 32, H * (D + 32) + 64
    sp = P * so + 4096
    pages = c.slots // P
    G = H if per_head else 1
    ssh, sso = 8, 8 * G + 16              # padded scale layout (bytes)
    ssp = P * sso + 64
    _say(f"dynamic padded per_head={per_head}")
    kc = torch.full((pages * sp,), 0xFF, dtype=torch.uint8, device=DEV)
    vc = torch.full_like(kc, 0xFF)
    ks = torch.full((pages * ssp,), 0xFF, dtype=torch.uint8, device=DEV)
    vs = torch.full_like(ks, 0xFF)
    st = run_dynamic(c, per_head, kc, vc, ks, vs, kc_strides=(sp, so, sh),
                     sc_strides=(ssp, sso, ssh if per_head else 0),
                     in_strides=(H * sh_in * 2, sh_in * 2), k_dev=to_dev(bk), v_dev=to_dev(bv))
    assert st == kv.OK
    okc = np.full(pages * sp, 0xFF, dtype=np.uint8)
    ovc = np.full_like(okc, 0xFF)
    oks = np.full(pages * ssp, 0xFF, dtype=np.uint8)
    ovs = np.full_like(oks, 0xFF)
    oracle.fp8_paged_dynamic(bk, bv, okc, ovc, c.indices, oks, ovs, src_dtype="bf16",
                             num_heads=H, head_dim=D, k_strides=(H * sh_in * 2, sh_in * 2),
                             v_strides=(H * sh_in * 2, sh_in * 2), kc_strides=(sp, so, sh),
                             vc_strides=(sp, so, sh), ks_strides=(ssp, sso, ssh if per_head else 0),
                             vs_strides=(ssp, sso, ssh if per_head else 0), per_head=per_head,
                             size_limit=c.slots, page_size=P)
    for got, want, nm in ((kc, okc, "k_cache"), (vc, ovc, "v_cache"), (ks, oks, "k_scales"),
                          (vs, ovs, "v_scales")):
        assert_cache_equal(got, want, nm)


def test_dynamic_out_of_range_indices():
    c = fp8_case(tokens=100, pages=8)
    limit = 384
    idx = np.random.Generator(np.random.PCG64(8)).permutation(limit)[:100].astype(np.int32)
    idx[10], idx[60] = -2, limit
    c.indices = idx
    kc = sentinel_cache(512, 1024)
    vc = sentinel_cache(512, 1024)
    ks = sentinel_cache(512, 32)
    vs = sentinel_cache(512, 32)
    _say("dynamic oob")
    assert run_dynamic(c, True, kc, vc, ks, vs, size_limit=limit) == kv.OK
    assert check_flag() == (kv.ERR_OOB, 10, 2)
    okc = np.full((512, 1024), 0xFF, dtype=np.uint8)
    ovc = np.full_like(okc, 0xFF)
    oks = np.full((512, 32), 0xFF, dtype=np.uint8)
    ovs = np.full_like(oks, 0xFF)
    st = oracle.fp8_paged_dynamic(c.k, c.v, okc, ovc, idx, oks, ovs, src_dtype="bf16",
                                  num_heads=8, head_dim=128, k_strides=(2048, 256),
                                  v_strides=(2048, 256), kc_strides=(64 * 1024, 1024, 128),
                                  vc_strides=(64 * 1024, 1024, 128), ks_strides=(64 * 32, 32, 4),
                                  vs_strides=(64 * 32, 32, 4), per_head=True, size_limit=limit,
                                  page_size=64)
    assert st == (98, 10, 2)
    for got, want, nm in ((kc, okc, "k_cache"), (vc, ovc, "v_cache"), (ks, oks, "k_scales"),
                          (vs, ovs, "v_scales")):
        assert_cache_equal(got, want, nm)


@pytest.mark.parametrize("per_head", [False, True])
def test_dynamic_tensor_api_flat_and_paged(per_head):
    c = fp8_case(tokens=200, pages=8)
    H, D, P = 8, 128, 64
    k3 = to_dev(c.k).view(torch.bfloat16).view(-1, H, D)
    v3 = to_dev(c.v).view(torch.bfloat16).view(-1, H, D)
    idx = to_dev(c.indices)
    okc, ovc, oks, ovs, _ = oracle.run_case_dynamic(c, per_head)
    for paged in (False, True):
        kc = sentinel_cache(c.slots, H * D)
        vc = sentinel_cache(c.slots, H * D)
        shape = (c.slots, H) if per_head else (c.slots,)
        ks = torch.full(shape, -1, dtype=torch.int32, device=DEV).view(torch.float32)
        vs = torch.full(shape, -1, dtype=torch.int32, device=DEV).view(torch.float32)
        if paged:
            kcv, vcv = kc.view(-1, P, H, D), vc.view(-1, P, H, D)
            ksv = ks.view(-1, P, *shape[1:])
            vsv = vs.view(-1, P, *shape[1:])
        else:
            kcv, vcv, ksv, vsv = kc.view(-1, H, D), vc.view(-1, H, D), ks, vs
        kv.store_kv_fp8_paged_dynamic(k3, v3, kcv, vcv, idx, ksv, vsv, per_head=per_head,
                                      page_size=P)
        np.testing.assert_array_equal(kc.cpu().numpy(), okc)
        np.testing.assert_array_equal(vc.cpu().numpy(), ovc)
        np.testing.assert_array_equal(ks.view(torch.int32).cpu().numpy().view(np.uint32).reshape(oks.shape), oks)
        np.testing.assert_array_equal(vs.view(torch.int32).cpu().numpy().view(np.uint32).reshape(ovs.shape), ovs)


@pytest.mark.parametrize("per_head", [False, True])
@pytest.mark.parametrize("tokens", [1, 2, 3, 5, 6, 7, 9, 13])
def test_dynamic_partial_blocks_and_bad_tokens(tokens, per_head):
    """Batches that leave the last block of waves partly empty, with a bad
    index at a different position of a block in each case: per token, the
    waves of a block hand their scales to one store, and every other token's
    row and scale must still land exactly, the bad token's not at all."""
    c = fp8_case(tokens=tokens, pages=2)
    limit = 100
    idx = np.random.Generator(np.random.PCG64(tokens)).permutation(limit)[:tokens].astype(np.int32)
    bad = {1: 0, 2: 1, 3: 2, 5: 4, 6: 1, 7: 5, 9: 8, 13: 6}[tokens]
    idx[bad] = limit + bad
    c.indices = idx
    kc = sentinel_cache(128, 1024)
    vc = sentinel_cache(128, 1024)
    G = 8 if per_head else 1
    ks = sentinel_cache(128, 4 * G)
    vs = sentinel_cache(128, 4 * G)
    _say(f"dynamic partial block per_head={per_head} T={tokens} bad={bad}")
    assert run_dynamic(c, per_head, kc, vc, ks, vs, size_limit=limit) == kv.OK
    assert check_flag() == (kv.ERR_OOB, bad, 1)
    okc = np.full((128, 1024), 0xFF, dtype=np.uint8)
    ovc = np.full_like(okc, 0xFF)
    oks = np.full((128, 4 * G), 0xFF, dtype=np.uint8)
    ovs = np.full_like(oks, 0xFF)
    st = oracle.fp8_paged_dynamic(c.k, c.v, okc, ovc, idx, oks, ovs, src_dtype="bf16",
                                  num_heads=8, head_dim=128, k_strides=(2048, 256),
                                  v_strides=(2048, 256), kc_strides=(64 * 1024, 1024, 128),
                                  vc_strides=(64 * 1024, 1024, 128),
                                  ks_strides=(64 * 4 * G, 4 * G, 4 if per_head else 0),
                                  vs_strides=(64 * 4 * G, 4 * G, 4 if per_head else 0),
                                  per_head=per_head, size_limit=limit, page_size=64)
    assert st == (tokens - 1, bad, 1)
    for got, want, nm in ((kc, okc, "k_cache"), (vc, ovc, "v_cache"), (ks, oks, "k_scales"),
                          (vs, ovs, "v_scales")):
        assert_cache_equal(got, want, nm)
