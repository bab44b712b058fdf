"""Seeded random store layouts, shared by the GPU parity test
(test_gpu_random.py) and its CPU bounds walk (test_random_layouts_walk.py).

Each draw_* function takes every random draw of one trial, in a fixed order,
and returns the layout with its host inputs; oracle_* runs the oracle over
host buffers of exactly the sizes the GPU test allocates on the device (an
input or cache buffer here has the byte length of its device twin), so an
oracle walk that stays inside them shows that the device buffers hold every
access of the same layout.  No torch, no GPU.
"""
import numpy as np

import oracle

OPS = ["copy", "fp8", "e5m2", "dynamic_token", "dynamic_head"]
SEEDS = range(120)


def rng_for(seed):
    return np.random.Generator(np.random.PCG64(90000 + seed))


def op_for(seed):
    return OPS[seed % len(OPS)]


def _indices(rng, T, limit, bad, dtype):
    assert limit >= T
    idx = rng.permutation(limit)[:T].astype(dtype)
    n_bad = int(bad * T)
    info = np.iinfo(dtype)
    choices = np.array([-1, limit, limit + 7, info.max, info.min], dtype=np.int64)
    for t in rng.choice(T, n_bad, replace=False) if n_bad else []:
        idx[t] = choices[rng.integers(0, choices.size)]
    return idx


def strided_indices(idx, stride):
    out = np.full(idx.size * stride, -3, dtype=idx.dtype)
    out[::stride] = idx
    return out


def draw_copy(rng):
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
    return dict(vw=vw, row=row, k_stride=k_stride, v_stride=v_stride, T=T, slots=slots,
                limit=limit, dtype=dtype, istride=istride, idx=idx, kb=kb, vb=vb, off=off,
                # device byte lengths: inputs at `off` inside T * stride + 64,
                # caches slots * row + 64 with the cache base at `off`
                k_in_bytes=T * k_stride + 64, v_in_bytes=T * v_stride + 64,
                cache_bytes=slots * row + 64)


def oracle_copy(L):
    okc = np.full(L["cache_bytes"], 0xFF, dtype=np.uint8)
    ovc = np.full_like(okc, 0xFF)
    ost = oracle.copy(L["kb"], L["vb"], okc[L["off"]:], ovc[L["off"]:], L["idx"],
                      row_bytes=L["row"], k_stride=L["k_stride"], v_stride=L["v_stride"],
                      cache_stride=L["row"], size_limit=L["limit"])
    return [okc, ovc], ost


def draw_fp8(rng, op):
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
    L = dict(op=op, dynamic=dynamic, per_head=per_head, D=D, H=H, src=src, T=T, P=P,
             pages=pages, limit=limit, dtype=dtype, istride=istride, idx=idx, kb=kb, vb=vb,
             k_in=(H * sh_in_k * 2, sh_in_k * 2), v_in=(H * sh_in_v * 2, sh_in_v * 2),
             kcs=kcs, vcs=vcs, ik=ik, iv=iv,
             kc_bytes=pages * kcs[0], vc_bytes=pages * vcs[0])
    if dynamic:
        G = H if per_head else 1

        def draw_scales():
            s_head = 4 + 4 * int(rng.integers(0, 2)) if per_head else 0
            s_off = G * max(s_head, 4) + 4 * int(rng.integers(0, 3))
            return (P * s_off + 4 * int(rng.integers(0, 5)), s_off, s_head)

        L["kss"], L["vss"] = draw_scales(), draw_scales()
        L["ks_bytes"], L["vs_bytes"] = pages * L["kss"][0] + 16, pages * L["vss"][0] + 16
    return L


def oracle_fp8(L):
    okc = np.full(L["kc_bytes"], 0xFF, dtype=np.uint8)
    ovc = np.full(L["vc_bytes"], 0xFF, dtype=np.uint8)
    common = dict(src_dtype=L["src"], num_heads=L["H"], head_dim=L["D"], k_strides=L["k_in"],
                  v_strides=L["v_in"], kc_strides=L["kcs"], vc_strides=L["vcs"],
                  size_limit=L["limit"], page_size=L["P"])
    if not L["dynamic"]:
        ost = oracle.fp8_paged(L["kb"], L["vb"], okc, ovc, L["idx"], inv_k_bits=L["ik"],
                               inv_v_bits=L["iv"], fmt="e5m2" if L["op"] == "e5m2" else "e4m3fn",
                               **common)
        return [okc, ovc], ost
    oks = np.full(L["ks_bytes"], 0xFF, dtype=np.uint8)
    ovs = np.full(L["vs_bytes"], 0xFF, dtype=np.uint8)
    ost = oracle.fp8_paged_dynamic(L["kb"], L["vb"], okc, ovc, L["idx"], oks, ovs,
                                   ks_strides=L["kss"], vs_strides=L["vss"],
                                   per_head=L["per_head"], **common)
    return [okc, ovc, oks, ovs], ost


def draw(seed):
    """(op, layout) of random trial `seed`."""
    rng, op = rng_for(seed), op_for(seed)
    return op, (draw_copy(rng) if op == "copy" else draw_fp8(rng, op))


def run_oracle(op, L):
    return oracle_copy(L) if op == "copy" else oracle_fp8(L)
