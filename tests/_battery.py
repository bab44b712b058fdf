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
    vb = np.ascontiguousarray(c.v).view(np.uint8)
    st = oracle.copy(kb, vb, kc, vc, strided, row_bytes=R, k_stride=c.in_stride_bytes,
                     v_stride=c.in_stride_bytes, cache_stride=R, size_limit=limit, idx_stride=2,
                     batch=40, lib=lib)
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
    sh_in = D + 8
    bk = np.full((T, H, sh_in), kvgen.PAD_POISON, dtype=np.uint16)
    bv = np.full_like(bk, kvgen.PAD_POISON)
    bk[:, :, :D] = c.k[keep].reshape(T, H, D)
    bv[:, :, :D] = c.v[keep].reshape(T, H, D)
    sh = D + 16
    so = H * sh + 32
    sp = P * so + 512
    pages = slots // P
    kc = np.full(pages * sp, 0xFF, dtype=np.uint8)
    vc = np.full_like(kc, 0xFF)
    st = oracle.fp8_paged(bk, bv, kc, vc, idx, src_dtype="bf16", num_heads=H, head_dim=D,
                          k_strides=(H * sh_in * 2, sh_in * 2), v_strides=(H * sh_in * 2, sh_in * 2),
                          kc_strides=(sp, so, sh), vc_strides=(sp, so, sh), size_limit=slots,
                          page_size=P, inv_k_bits=c.inv_k_bits, inv_v_bits=c.inv_v_bits, lib=lib)
    if st != (T, -1, 0):
        return False
    ok = True
    for cache, src, inv in ((kc, c.k[keep], c.inv_k_bits), (vc, c.v[keep], c.inv_v_bits)):
        view = np.lib.stride_tricks.as_strided(cache, shape=(pages, P, H, D), strides=(sp, so, sh, 1))
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
