"""A fast subset of the oracle pins, runnable against any build of the oracle.

``python -m tests._battery <liboracle.so>`` exits 0 when every check passes and
1 otherwise (printing the failing checks).  The mutation test runs it against
oracle builds with planted mistakes, in a child process each, so that a
mutant that writes out of bounds cannot take the test run down with it.
"""
import sys

import numpy as np

import kvgen
import oracle
from tests import _ref

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _pins(lib):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_pins.txt")
    ys, cs = [], []
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            a, b = line.split()[:2]
            ys.append(int(a, 16))
            cs.append(int(b, 16))
    y = np.array(ys, dtype=np.uint32).view(np.float32)
    return np.array_equal(oracle.e4m3fn(y, lib=lib), np.array(cs, dtype=np.uint8))


def _exhaustive(lib, src, inv):
    return np.array_equal(oracle.quantize(ALL16, src, inv, lib=lib),
                          _ref.expected_codes(ALL16, src, inv))


def _copy(lib):
    c = kvgen.workload(5, tokens=40, slots=128)          # strided fp16 input rows
    R = c.row_bytes
    limit = 100
    idx = np.random.Generator(np.random.PCG64(1)).permutation(limit)[:40].astype(np.int64)
    idx[7] = limit                                        # two rejected rows
    idx[30] = -1
    strided = np.full(idx.size * 2, 3, dtype=np.int64)
    strided[::2] = idx
    kc = np.full((128, R), 0xFF, dtype=np.uint8)
    vc = np.full_like(kc, 0xFF)
    kb = np.ascontiguousarray(c.k).view(np.uint8)
    # V rows at their own stride (64 bytes wider than K's), padding poisoned
    vb = np.full((40, c.in_stride_bytes + 64), 0xAB, dtype=np.uint8)
    vb[:, :c.in_stride_bytes] = np.ascontiguousarray(c.v).view(np.uint8)
    st = oracle.copy(kb, vb, kc, vc, strided, row_bytes=R, k_stride=c.in_stride_bytes,
                     v_stride=c.in_stride_bytes + 64, cache_stride=R, size_limit=limit,
                     idx_stride=2, batch=40, lib=lib)
    good = [t for t in range(40) if t not in (7, 30)]
    return (st == (38, 7, 2) and np.all(kc[limit:] == 0xFF)
            and np.array_equal(kc[idx[good]], kb[good, :R])
            and np.array_equal(vc[idx[good]], vb[good, :R])
            and int((kc[:limit] != 0xFF).any(axis=1).sum()) == 38)


def _fp8(lib):
    c = kvgen.workload(4, tokens=100, slots=4 * 64)
    H, D, P = c.num_heads, c.head_dim, 48
    slots = (c.slots // P) * P
    keep = c.indices < slots
    idx = c.indices[keep].copy()
    T = idx.size
    # K and V each with their own input head padding and cache layout
    sh_in, sh_in_v = D + 8, D + 24
    bk = np.full((T, H, sh_in), kvgen.PAD_POISON, dtype=np.uint16)
    bv = np.full((T, H, sh_in_v), kvgen.PAD_POISON, dtype=np.uint16)
    bk[:, :, :D] = c.k[keep].reshape(T, H, D)
    bv[:, :, :D] = c.v[keep].reshape(T, H, D)
    sh, sh_v = D + 16, D + 48
    so, so_v = H * sh + 32, H * sh_v + 16
    sp, sp_v = P * so + 512, P * so_v + 256
    pages = slots // P
    kc = np.full(pages * sp, 0xFF, dtype=np.uint8)
    vc = np.full(pages * sp_v, 0xFF, dtype=np.uint8)
    st = oracle.fp8_paged(bk, bv, kc, vc, idx, src_dtype="bf16", num_heads=H, head_dim=D,
                          k_strides=(H * sh_in * 2, sh_in * 2),
                          v_strides=(H * sh_in_v * 2, sh_in_v * 2),
                          kc_strides=(sp, so, sh), vc_strides=(sp_v, so_v, sh_v), size_limit=slots,
                          page_size=P, inv_k_bits=c.inv_k_bits, inv_v_bits=c.inv_v_bits, lib=lib)
    if st != (T, -1, 0):
        return False
    ok = True
    for cache, src, inv, (cp, co, ch) in ((kc, c.k[keep], c.inv_k_bits, (sp, so, sh)),
                                          (vc, c.v[keep], c.inv_v_bits, (sp_v, so_v, sh_v))):
        view = np.lib.stride_tricks.as_strided(cache, shape=(pages, P, H, D), strides=(cp, co, ch, 1))
        loc = idx.astype(np.int64)
        got = view[loc // P, loc % P].reshape(T, H * D)
        ok &= np.array_equal(got, _ref.expected_codes(src, "bf16", inv))
    return bool(ok)


def _dynamic(lib):
    c = kvgen.workload(4, tokens=60, slots=2 * 64)
    c.k[3, :] = 0                                       # an all-zero group
    ok = True
    for per_head in (False, True):
        kc, vc, ks, vs, st = oracle.run_case_dynamic(c, per_head, lib=lib)
        idx = c.indices.astype(np.int64)
        for cache, scales, src in ((kc, ks, c.k), (vc, vs, c.v)):
            codes, sc = _ref.dynamic_expected(src, "bf16", 8, 128, per_head)
            ok &= st == (60, -1, 0) and np.array_equal(cache[idx], codes) \
                and np.array_equal(scales[idx], sc.view(np.uint32))
    return bool(ok)


def _dynamic_layouts(lib):
    """Per-head dynamic scales with K and V in different layouts: V input heads
    padded, V cache slots and heads padded, V scales at their own strides."""
    c = kvgen.workload(4, tokens=60, slots=2 * 64)
    H, D, P, T = 8, 128, 64, 60
    slots = c.slots
    idx = c.indices.astype(np.int64)
    shv = D + 16
    bv = np.full((T, H, shv), kvgen.PAD_POISON, dtype=np.uint16)
    bv[:, :, :D] = c.v.reshape(T, H, D)
    kc = np.full((slots, H * D), 0xFF, dtype=np.uint8)
    vsh, vso = D + 32, H * (D + 32) + 64
    vc = np.full(slots * vso, 0xFF, dtype=np.uint8)
    ks = np.full((slots, H), 0xFFFFFFFF, dtype=np.uint32)
    vs = np.full((slots, 2 * H), 0xFFFFFFFF, dtype=np.uint32)   # V: head stride 8 bytes
    st = oracle.fp8_paged_dynamic(
        c.k, bv, kc, vc, c.indices, ks, vs, src_dtype="bf16", num_heads=H, head_dim=D,
        k_strides=(H * D * 2, D * 2), v_strides=(H * shv * 2, shv * 2),
        kc_strides=(P * H * D, H * D, D), vc_strides=(P * vso, vso, vsh),
        ks_strides=(P * H * 4, H * 4, 4), vs_strides=(P * 2 * H * 4, 2 * H * 4, 8),
        per_head=True, size_limit=slots, page_size=P, lib=lib)
    codes_k, sc_k = _ref.dynamic_expected(c.k, "bf16", H, D, True)
    codes_v, sc_v = _ref.dynamic_expected(c.v, "bf16", H, D, True)
    vview = np.lib.stride_tricks.as_strided(vc, shape=(slots, H, D), strides=(vso, vsh, 1))
    return bool(st == (T, -1, 0) and np.array_equal(kc[idx], codes_k)
                and np.array_equal(vview[idx].reshape(T, H * D), codes_v)
                and np.array_equal(ks[idx], sc_k.view(np.uint32))
                and np.array_equal(vs[idx][:, ::2], sc_v.view(np.uint32))
                and np.all(vs[:, 1::2] == 0xFFFFFFFF))


def _decode(lib, src):
    got = np.array([lib.oracle_src_to_float(int(b), int(src == "fp16")) for b in ALL16],
                   dtype=np.float32)
    want = _ref.src_bits_to_f32(ALL16, src)
    nan = np.isnan(want)
    return (np.array_equal(np.isnan(got), nan)
            and np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32)))


def _e5m2(lib):
    y, want = [], []
    import os
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "e5m2_pins.txt")):
        if line.strip() and not line.startswith("#"):
            a, b = line.split()[:2]
            y.append(int(a, 16))
            want.append(int(b, 16))
    yv = np.array(y, dtype=np.uint32).view(np.float32)
    return (np.array_equal(oracle.e5m2(yv, lib=lib), np.array(want, dtype=np.uint8))
            and np.array_equal(oracle.quantize(ALL16, "fp16", kvgen.INV_K_BITS, lib=lib, fmt="e5m2"),
                               _ref.expected_codes(ALL16, "fp16", kvgen.INV_K_BITS, "e5m2")))


CHECKS = {
    "decode_bf16": lambda lib: _decode(lib, "bf16"),
    "decode_fp16": lambda lib: _decode(lib, "fp16"),
    "golden_pins": _pins,
    "exhaustive_bf16_inv_k": lambda lib: _exhaustive(lib, "bf16", kvgen.INV_K_BITS),
    "exhaustive_fp16_noscale": lambda lib: _exhaustive(lib, "fp16", None),
    "copy_store": _copy,
    "fp8_store": _fp8,
    "fp8_dynamic": _dynamic,
    "fp8_dynamic_layouts": _dynamic_layouts,
    "e5m2": _e5m2,
}


def run(lib_path):
    lib = oracle.load(lib_path)
    failed = []
    for name, fn in CHECKS.items():
        try:
            if not fn(lib):
                failed.append(name)
        except Exception as e:  # a mutant may also raise
            failed.append(f"{name} ({type(e).__name__})")
    return failed


if __name__ == "__main__":
    failed = run(sys.argv[1])
    print("FAILED:" if failed else "ALL PASSED", ", ".join(failed))
    sys.exit(1 if failed else 0)
