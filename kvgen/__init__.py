"""Seeded synthetic inputs for the KV-cache store.

This module only *creates inputs*: random K/V rows, index tensors and the
fixed inverse-scale bit patterns.  It contains none of the store's arithmetic
(no addressing, no quantisation) and is the single source of inputs that both
the CPU oracle and the HIP path consume, so that both see identical bits.

Everything is numpy on the host, driven by ``numpy.random.PCG64`` with a
fixed seed per workload (seed = 1000 + workload number).  Values are returned
as raw bit patterns (``uint16`` for bf16/fp16 elements, ``int32``/``int64`` for
indices) so that no consumer can round them differently.

Workloads (shapes follow the two store variants on the pages: the sglang
``kvcache.cuh`` scatter-copy, section "store_kvcache", and the sglang
``trtllm_fp8_kv_kernel.py`` fused FP8 paged write, "fused_fp8_set_kv_buffer"):

1. tiny copy     16 tok, 2x64 bf16, int32, 256 slots
2. decode copy   256 tok, 8x128 bf16, int64, 2^20 slots
3. prefill copy  32768 tok, 8x128 bf16, int32, 2^21 slots in 16-slot pages
4. fp8 paged     16384 tok, 8x128 bf16 (0.1% outliers x50), int32, page 64,
                 2^21 slots, inverse scales 1/2.5 and 1/1.7 (fp32)
5. wide strided  8192 tok, 1x576 fp16, input row stride 640, int64, 2^19 slots
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16 = "bf16"
FP16 = "fp16"
I32 = "i32"
I64 = "i64"

# fp32 bit patterns of 1.0f/2.5f and 1.0f/1.7f, i.e. the fp32 reciprocal of the
# fp32 scale computed in fp32 (the fused kernel's wrapper inverts the scale on
# the device in fp32 before the launch).
INV_K_BITS = 0x3ECCCCCD
INV_V_BITS = 0x3F169696
# Poison written into the padding columns of strided inputs (an fp16 NaN); it
# must never reach a cache.
PAD_POISON = 0x7E00
# Byte used to fill caches before a store: 0xFF is a NaN in bf16, fp16 and
# e4m3fn, so no finite input can produce it.
SENTINEL = 0xFF


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def f32_to_bits(x) -> int:
    return int(np.asarray(x, dtype=np.float32).view(np.uint32))


def _round_f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _round_f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    return _round_f32_to_bf16_bits(x) if dtype == BF16 else _round_f32_to_f16_bits(x)


def perm_prefix_indices(rng: np.random.Generator, slots: int, n: int) -> np.ndarray:
    """``n`` distinct slots: a prefix of a uniform random permutation of the slots."""
    if n > slots:
        raise ValueError("more tokens than slots")
    return rng.permutation(slots)[:n].astype(np.int64)


def paged_run_indices(rng: np.random.Generator, slots: int, page: int, n: int) -> np.ndarray:
    """Consecutive runs inside randomly permuted free pages.

    ``perm`` is a permutation of the page ids; token t goes to slot
    ``perm[t // page] * page + t % page``, so each page is filled front to back.
    """
    if slots % page:
        raise ValueError("slots must be a multiple of the page size")
    pages_needed = -(-n // page)
    if pages_needed > slots // page:
        raise ValueError("more tokens than slots")
    perm = rng.permutation(slots // page)[:pages_needed].astype(np.int64)
    t = np.arange(n, dtype=np.int64)
    return perm[t // page] * page + t % page


@dataclass
class Case:
    """One store workload, as raw bits plus the layout facts a caller passes."""
    name: str
    kind: str                 # "copy" or "fp8"
    src_dtype: str            # bf16 / fp16
    num_tokens: int
    num_heads: int
    head_dim: int
    in_stride_elems: int      # input row stride in elements (>= heads*dim)
    k: np.ndarray             # uint16 [T, in_stride_elems]
    v: np.ndarray             # uint16 [T, in_stride_elems]
    indices: np.ndarray       # int32 / int64 [T]
    idx_dtype: str
    slots: int                # cache rows (slots); also the bound on indices
    page_size: int = 1
    inv_k_bits: Optional[int] = None
    inv_v_bits: Optional[int] = None
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def row_elems(self) -> int:
        return self.num_heads * self.head_dim

    @property
    def row_bytes(self) -> int:
        return self.row_elems * 2

    @property
    def in_stride_bytes(self) -> int:
        return self.in_stride_elems * 2

    @property
    def idx_bytes(self) -> int:
        return 4 if self.idx_dtype == I32 else 8

    @property
    def cache_row_bytes(self) -> int:
        """Bytes one slot occupies in the cache (bf16/fp16 copy or fp8)."""
        return self.row_bytes if self.kind == "copy" else self.row_elems

    def algorithmic_bytes(self) -> int:
        """Bytes the store must move: K/V rows read, indices read, cache rows
        written (+ the two fp32 inverse scales for the fp8 store)."""
        t = self.num_tokens
        b = 2 * t * self.row_bytes + t * self.idx_bytes + 2 * t * self.cache_row_bytes
        if self.kind == "fp8":
            b += 4 * ((self.inv_k_bits is not None) + (self.inv_v_bits is not None))
        return b


def _make(name, kind, seed, T, H, D, src_dtype, idx_dtype, slots, *, page_size=1,
          index_scheme="perm", index_page=1, in_stride_elems=None, outlier_p=0.0,
          outlier_mul=1.0, inv_k_bits=None, inv_v_bits=None) -> Case:
    rng = np.random.Generator(np.random.PCG64(seed))
    row = H * D
    stride = in_stride_elems or row
    if index_scheme == "perm":
        idx = perm_prefix_indices(rng, slots, T)
    elif index_scheme == "paged":
        idx = paged_run_indices(rng, slots, index_page, T)
    else:
        raise ValueError(index_scheme)
    bufs = []
    for _ in range(2):
        x = rng.standard_normal((T, row), dtype=np.float32)
        if outlier_p > 0.0:
            hit = rng.random((T, row)) < outlier_p
            x = np.where(hit, x * np.float32(outlier_mul), x).astype(np.float32)
        buf = np.full((T, stride), PAD_POISON, dtype=np.uint16)
        buf[:, :row] = _to_bits(x, src_dtype)
        bufs.append(buf)
    idx = idx.astype(np.int32 if idx_dtype == I32 else np.int64)
    return Case(name=name, kind=kind, src_dtype=src_dtype, num_tokens=T, num_heads=H, head_dim=D,
                in_stride_elems=stride, k=bufs[0], v=bufs[1], indices=idx, idx_dtype=idx_dtype,
                slots=slots, page_size=page_size, inv_k_bits=inv_k_bits, inv_v_bits=inv_v_bits,
                seed=seed, extra={"index_page": index_page})


WORKLOADS = {
    1: dict(name="tiny_copy", kind="copy", T=16, H=2, D=64, src_dtype=BF16, idx_dtype=I32,
            slots=256, index_scheme="perm"),
    2: dict(name="decode_copy", kind="copy", T=256, H=8, D=128, src_dtype=BF16, idx_dtype=I64,
            slots=1 << 20, index_scheme="perm"),
    3: dict(name="prefill_copy", kind="copy", T=32768, H=8, D=128, src_dtype=BF16, idx_dtype=I32,
            slots=1 << 21, index_scheme="paged", index_page=16),
    4: dict(name="fp8_paged", kind="fp8", T=16384, H=8, D=128, src_dtype=BF16, idx_dtype=I32,
            slots=1 << 21, page_size=64, index_scheme="paged", index_page=64,
            outlier_p=0.001, outlier_mul=50.0,
            inv_k_bits=INV_K_BITS, inv_v_bits=INV_V_BITS),
    5: dict(name="wide_strided_copy", kind="copy", T=8192, H=1, D=576, src_dtype=FP16,
            idx_dtype=I64, slots=1 << 19, index_scheme="perm", in_stride_elems=640),
}


def workload(n: int, *, tokens: Optional[int] = None, slots: Optional[int] = None,
             seed: Optional[int] = None) -> Case:
    """Workload ``n`` (1..5) at full size, or with fewer tokens / slots for
    quick runs (same recipe, same structure)."""
    spec = dict(WORKLOADS[n])
    name = spec.pop("name")
    kind = spec.pop("kind")
    T = tokens if tokens is not None else spec.pop("T")
    spec.pop("T", None)
    if slots is not None:
        spec["slots"] = slots
    return _make(name, kind, 1000 + n if seed is None else seed, T=T, **spec)


def disjoint_index_sets(case: Case, count: int, seed: Optional[int] = None) -> list:
    """``count`` index arrays for ``case`` over pairwise-disjoint slots, used to
    rotate through memory when timing.  Set 0 is the workload's own index
    array; the others are drawn by the same scheme from the slots (or pages)
    that set 0 leaves free."""
    rng = np.random.Generator(np.random.PCG64((case.seed if seed is None else seed) + 7919))
    T = case.num_tokens
    dt = case.indices.dtype
    first = case.indices.astype(np.int64)
    page = case.extra.get("index_page", 1)
    out = [case.indices.copy()]
    if page > 1:
        need = -(-T // page)
        used = np.unique(first // page)
        free = np.setdiff1d(np.arange(case.slots // page, dtype=np.int64), used)
        if need * (count - 1) > free.size:
            raise ValueError("not enough pages for disjoint sets")
        perm = rng.permutation(free)
        t = np.arange(T, dtype=np.int64)
        for s in range(count - 1):
            p = perm[s * need:(s + 1) * need]
            out.append((p[t // page] * page + t % page).astype(dt))
        return out
    free = np.setdiff1d(np.arange(case.slots, dtype=np.int64), first)
    if T * (count - 1) > free.size:
        raise ValueError("not enough slots for disjoint sets")
    perm = rng.permutation(free)
    out += [perm[s * T:(s + 1) * T].astype(dt) for s in range(count - 1)]
    return out


def all_patterns_case(src_dtype: str, inv_k_bits=None, inv_v_bits=None) -> Case:
    """Every 16-bit pattern once: 64 tokens x (8 heads x 128 dims), K holds the
    patterns in order and V holds them reversed.  Index t -> slot t, page 64."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(64, 1024)
    k = pats.copy()
    v = pats[::-1, ::-1].copy()
    idx = np.arange(64, dtype=np.int32)
    return Case(name=f"all_{src_dtype}", kind="fp8", src_dtype=src_dtype, num_tokens=64,
                num_heads=8, head_dim=128, in_stride_elems=1024, k=k, v=v, indices=idx,
                idx_dtype=I32, slots=128, page_size=64, inv_k_bits=inv_k_bits,
                inv_v_bits=inv_v_bits, seed=0)


DEST_PATTERNS = ("contiguous", "runs16_in_64MiB", "workload", "single_slots")


def pattern_index_sets(case: Case, pattern: str, count: int, seed: int = 4242) -> list:
    """``count`` pairwise-disjoint index arrays for ``case`` that send its
    tokens to the cache in one of four destination patterns, to take apart
    what the destination layout costs a store (the rows, token order and
    index type stay those of the case):

    * ``contiguous``: set s stores to slots [s*T, (s+1)*T);
    * ``runs16_in_64MiB``: 16-slot runs in random page order, each set inside
      its own extent of T slots (64 MiB for 2 KiB rows);
    * ``workload``: the case's own scheme (``disjoint_index_sets``);
    * ``single_slots``: single slots drawn uniformly over the whole cache.
    """
    T, dt = case.num_tokens, case.indices.dtype
    if pattern == "workload":
        return disjoint_index_sets(case, count)
    if count * T > case.slots:
        raise ValueError("not enough slots for disjoint sets")
    rng = np.random.Generator(np.random.PCG64(seed))
    if pattern == "contiguous":
        return [np.arange(s * T, (s + 1) * T, dtype=np.int64).astype(dt) for s in range(count)]
    if pattern == "runs16_in_64MiB":
        if T % 16:
            raise ValueError("token count must be a multiple of 16")
        pages = T // 16
        t = np.arange(T, dtype=np.int64)
        out = []
        for s in range(count):
            perm = rng.permutation(pages).astype(np.int64) + s * pages
            out.append((perm[t // 16] * 16 + t % 16).astype(dt))
        return out
    if pattern == "single_slots":
        pick = rng.permutation(case.slots)[:count * T].astype(np.int64)
        return [pick[s * T:(s + 1) * T].astype(dt) for s in range(count)]
    raise ValueError(f"unknown destination pattern {pattern!r}")


EXTENT_MIB = (64, 128, 256, 512, 1024, 2048, 4096)


def extent_index_sets(case: Case, extent_bytes: int, count: int, seed: int = 4343) -> list:
    """``count`` pairwise-disjoint index arrays for ``case`` that keep its
    scheme (runs of ``index_page`` consecutive slots, whole runs in random
    order) but draw each set's runs from a cache extent of ``extent_bytes``
    per tensor, to see how the store's time depends on how densely the
    written runs sit in memory.  While ``count`` extents fit in the cache and
    one extent is smaller than the runs of all sets together, set s takes
    its runs from its own extent [s*E, (s+1)*E); otherwise the sets share the
    extent [0, E), each with its own runs."""
    run = case.extra.get("index_page", 1)
    T, dt = case.num_tokens, case.indices.dtype
    need = -(-T // run)
    ext_runs = extent_bytes // (run * case.row_bytes)
    all_runs = case.slots // run
    own = ext_runs * count <= all_runs and ext_runs < need * count
    if ext_runs < need or (not own and (need * count > ext_runs or ext_runs > all_runs)):
        raise ValueError("extent does not fit the sets")
    rng = np.random.Generator(np.random.PCG64(seed))
    t = np.arange(T, dtype=np.int64)
    out = []
    shared = None if own else rng.permutation(ext_runs)
    for s in range(count):
        if own:
            p = rng.permutation(ext_runs)[:need].astype(np.int64) + s * ext_runs
        else:
            p = shared[s * need:(s + 1) * need].astype(np.int64)
        out.append((p[t // run] * run + t % run).astype(dt))
    return out
