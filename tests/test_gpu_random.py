"""Seeded randomized parity: every store entry point over random layouts.

Each trial draws (from a fixed seed) the operation, token count, heads and
head size, input and cache paddings, page size, index type and stride, scales
and a few out-of-range indices, runs the library through its C ABI and the
oracle on the same bytes, and compares every byte of every output buffer and
the error flag.  The trials are fixed by their seeds, so a failure names a
reproducible case.
"""
import numpy as np
import pytest
import torch

import fp8_kv_quantization_amd as kv
import oracle
from tests._gpu import DEV, assert_cache_equal, check_flag, stream

pytestmark = pytest.mark.gpu

OPS = ["copy", "fp8", "e5m2", "dynamic_token", "dynamic_head"]


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _indices(rng, T, limit, bad, dtype):
    assert limit >= T
    idx = rng.permutation(limit)[:T].astype(dtype)
    n_bad = int(bad * T)
    info = np.iinfo(dtype)
    choices = np.array([-1, limit, limit + 7, info.max, info.min], dtype=np.int64)
    for t in rng.choice(T, n_bad, replace=False) if n_bad else []:
        idx[t] = choices[rng.integers(0, choices.size)]
    return idx


def _strided_indices(rng, idx, stride):
    out = np.full(idx.size * stride, -3, dtype=idx.dtype)
    out[::stride] = idx
    return out


def trial_copy(rng):
    vw = int(rng.choice([4, 8, 16]))
    row = int(rng.integers(1, 700)) * 4
    row -= row % vw
    row = max(row, vw)
    k_stride = row + int(rng.integers(0, 4)) * vw        # K and V rows at their own strides
    v_stride = row + int(rng.integers(0, 4)) * vw
    T = int(rng.integers(1, 1500))
    slots = T + int(rng.integers(2, 400))
    limit = slots - int(rng.integers(0, 3))          # >= T: every token has an index
    dtype = np.int64 if rng.integers(0, 2) else np.int32
    istride = int(rng.integers(1, 4))
    idx = _indices(rng, T, limit, float(rng.choice([0.0, 0.0, 0.02])), dtype)
    kb = rng.integers(0, 256, (T, k_stride), dtype=np.uint8)
    vb = rng.integers(0, 256, (T, v_stride), dtype=np.uint8)
    off = int(rng.choice([0, vw]))
    _say(f"copy row={row} strides={k_stride},{v_stride} T={T} slots={slots} limit={limit} "
         f"vw={vw} {dtype.__name__} istride={istride} off={off}")
    kd = torch.zeros(T * k_stride + 64, dtype=torch.uint8, device=DEV)
    vd = torch.zeros(T * v_stride + 64, dtype=torch.uint8, device=DEV)
    kd[off:off + T * k_stride] = _dev(kb.reshape(-1))
    vd[off:off + T * v_stride] = _dev(vb.reshape(-1))
    kc = torch.full((slots * row + 64,), 0xFF, dtype=torch.uint8, device=DEV)
    vc = torch.full_like(kc, 0xFF)
    di = _dev(_strided_indices(rng, idx, istride))
    st = kv.kvstore_copy(kd.data_ptr() + off, vd.data_ptr() + off, kc.data_ptr() + off,
                         vc.data_ptr() + off, di.data_ptr(),
                         kv.IDX_I64 if dtype == np.int64 else kv.IDX_I32, istride, row, k_stride,
                         v_stride, row, T, limit, stream())
    assert st == kv.OK
    okc = np.full(slots * row + 64, 0xFF, dtype=np.uint8)
    ovc = np.full_like(okc, 0xFF)
    ost = oracle.copy(kb, vb, okc[off:], ovc[off:], idx, row_bytes=row, k_stride=k_stride,
                      v_stride=v_stride, cache_stride=row, size_limit=limit)
    return [(kc, okc), (vc, ovc)], ost


def trial_fp8(rng, op):
    dynamic = op.startswith("dynamic")
    per_head = op == "dynamic_head"
    if per_head:
        D = int(rng.choice([16, 32, 64, 128, 256]))
        H = int(rng.integers(1, max(2, 4096 // D // 2) + 1))
    else:
        D = int(rng.integers(1, 17)) * 16
        # static stores up to 24 heads (up to 6144 elements: rows split over
        # grid slices); dynamic scales keep the whole row in one wave
        H = int(rng.integers(1, 25)) if not dynamic else min(int(rng.integers(1, 9)), 4096 // D)
    src = "fp16" if rng.integers(0, 2) else "bf16"
    T = int(rng.integers(1, 800))
    P = int(rng.choice([1, 3, 16, 48, 64, 100]))
    pages = (T + int(rng.integers(0, 300))) // P + 1
    slots = pages * P
    limit = slots - int(rng.integers(0, 2))
    dtype = np.int64 if rng.integers(0, 2) else np.int32
    istride = int(rng.integers(1, 3))
    idx = _indices(rng, T, limit, float(rng.choice([0.0, 0.0, 0.03])), dtype)
    # K and V each: input [T, H, D + in_pad] elements, cache [pages, P, H, D +
    # c_pad] bytes + page padding, padding drawn separately for K and V
    scale_mag = np.float32(rng.choice([1.0, 30.0, 3000.0]))

    def draw_input():
        sh_in = D + int(rng.choice([0, 8, 16]))
        raw_bits = rng.integers(0, 65536, (T, H, sh_in), dtype=np.uint32).astype(np.uint16)
        # mostly ordinary magnitudes, some raw patterns (NaN / inf / subnormal)
        ordinary = rng.standard_normal((T, H, sh_in)).astype(np.float32) * scale_mag
        if src == "bf16":
            u = ordinary.view(np.uint32)
            ob = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        else:
            ob = ordinary.astype(np.float16).view(np.uint16)
        raw = rng.random((T, H, sh_in)) < 0.01
        return np.where(raw, raw_bits, ob).astype(np.uint16), sh_in

    def draw_cache():
        sh = D + int(rng.choice([0, 16, 32]))
        so = H * sh + int(rng.choice([0, 0, 16]))
        return (P * so + int(rng.choice([0, 16, 4096])), so, sh)

    kb, sh_in_k = draw_input()
    vb, sh_in_v = draw_input()
    kcs, vcs = draw_cache(), draw_cache()
    scales = [None, 0x3ECCCCCD, 0x3F169696, 0x41200000, 0x3A83126F]
    ik = scales[int(rng.integers(0, len(scales)))]
    iv = scales[int(rng.integers(0, len(scales)))]
    _say(f"{op} T={T} H={H} D={D} src={src} P={P} pages={pages} limit={limit} "
         f"{dtype.__name__} istride={istride} in={sh_in_k},{sh_in_v} kc={kcs} vc={vcs} "
         f"ik={ik} iv={iv}")
    kd, vd = _dev(kb), _dev(vb)
    kc = torch.full((pages * kcs[0],), 0xFF, dtype=torch.uint8, device=DEV)
    vc = torch.full((pages * vcs[0],), 0xFF, dtype=torch.uint8, device=DEV)
    di = _dev(_strided_indices(rng, idx, istride))
    okc = np.full(pages * kcs[0], 0xFF, dtype=np.uint8)
    ovc = np.full(pages * vcs[0], 0xFF, dtype=np.uint8)
    k_in = (H * sh_in_k * 2, sh_in_k * 2)
    v_in = (H * sh_in_v * 2, sh_in_v * 2)
    idt = kv.IDX_I64 if dtype == np.int64 else kv.IDX_I32
    sdt = kv.SRC_FP16 if src == "fp16" else kv.SRC_BF16
    if not dynamic:
        ikd = _dev(np.array([ik], dtype=np.uint32).view(np.float32)) if ik is not None else None
        ivd = _dev(np.array([iv], dtype=np.uint32).view(np.float32)) if iv is not None else None
        entry = kv.kvstore_fp8_paged_e5m2 if op == "e5m2" else kv.kvstore_fp8_paged
        st = entry(kd.data_ptr(), vd.data_ptr(), kc.data_ptr(), vc.data_ptr(), di.data_ptr(), idt,
                   istride, sdt, H, D, *k_in, *v_in, *kcs, *vcs, T, limit, P,
                   None if ikd is None else ikd.data_ptr(), None if ivd is None else ivd.data_ptr(),
                   stream())
        torch.cuda.synchronize()
        assert st == kv.OK
        ost = oracle.fp8_paged(kb, vb, okc, ovc, idx, src_dtype=src, num_heads=H, head_dim=D,
                               k_strides=k_in, v_strides=v_in, kc_strides=kcs, vc_strides=vcs,
                               size_limit=limit, page_size=P, inv_k_bits=ik, inv_v_bits=iv,
                               fmt="e5m2" if op == "e5m2" else "e4m3fn")
        return [(kc, okc), (vc, ovc)], ost
    G = H if per_head else 1

    def draw_scales():
        s_head = 4 + 4 * int(rng.integers(0, 2)) if per_head else 0
        s_off = G * max(s_head, 4) + 4 * int(rng.integers(0, 3))
        return (P * s_off + 4 * int(rng.integers(0, 5)), s_off, s_head)

    kss, vss = draw_scales(), draw_scales()
    ks = torch.full((pages * kss[0] + 16,), 0xFF, dtype=torch.uint8, device=DEV)
    vs = torch.full((pages * vss[0] + 16,), 0xFF, dtype=torch.uint8, device=DEV)
    oks = np.full(pages * kss[0] + 16, 0xFF, dtype=np.uint8)
    ovs = np.full(pages * vss[0] + 16, 0xFF, dtype=np.uint8)
    st = kv.kvstore_fp8_paged_dynamic(
        kd.data_ptr(), vd.data_ptr(), kc.data_ptr(), vc.data_ptr(), di.data_ptr(), idt, istride,
        sdt, H, D, *k_in, *v_in, *kcs, *vcs, ks.data_ptr(), vs.data_ptr(),
        kv.SCALE_PER_TOKEN_HEAD if per_head else kv.SCALE_PER_TOKEN, *kss, *vss, T, limit, P,
        stream())
    torch.cuda.synchronize()
    assert st == kv.OK
    ost = oracle.fp8_paged_dynamic(kb, vb, okc, ovc, idx, oks, ovs, src_dtype=src, num_heads=H,
                                   head_dim=D, k_strides=k_in, v_strides=v_in, kc_strides=kcs,
                                   vc_strides=vcs, ks_strides=kss, vs_strides=vss,
                                   per_head=per_head, size_limit=limit, page_size=P)
    return [(kc, okc), (vc, ovc), (ks, oks), (vs, ovs)], ost


@pytest.mark.parametrize("seed", range(60))
def test_random_layouts(seed):
    rng = np.random.Generator(np.random.PCG64(90000 + seed))
    op = OPS[seed % len(OPS)]
    check_flag()
    if op == "copy":
        pairs, ost = trial_copy(rng)
    else:
        pairs, ost = trial_fp8(rng, op)
    _, first_bad, bad_count = ost
    st, fb, bc = check_flag()
    assert (fb, bc) == (first_bad, bad_count)
    assert st == (kv.ERR_OOB if bad_count else kv.OK)
    for i, (got, want) in enumerate(pairs):
        assert_cache_equal(got, want, f"buffer {i}")
