"""Independent test-side references used to pin the oracle.

Nothing here is shared with the oracle or with the HIP library.  The e4m3fn
table is decoded from the format definition (1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits, code S.1111.111 is NaN, no infinities), and the
encoder is a brute-force nearest-value search over that table; input decoding
and the fp32 multiply use library routines (torch's bfloat16, numpy's float16
and float32).
"""
from __future__ import annotations

import numpy as np
import torch


def e4m3fn_decode(code: int) -> float:
    """Value of an e4m3fn code, from the format definition."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# Non-negative finite values, indexed by code 0x00..0x7E.
TABLE = np.array([e4m3fn_decode(c) for c in range(0x7F)], dtype=np.float64)


def e5m2_decode(code: int) -> float:
    """Value of an e5m2 code, from the format definition (1 sign, 5 exponent
    bits with bias 15, 2 mantissa bits; exponent 31 is inf / NaN)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 2) & 0x1F
    m = code & 0x3
    if e == 0x1F:
        return s * float("inf") if m == 0 else float("nan")
    if e == 0:
        return s * m * 2.0 ** -16
    return s * (1.0 + m / 4.0) * 2.0 ** (e - 15)


# Non-negative finite e5m2 values, indexed by code 0x00..0x7B.
TABLE_E5M2 = np.array([e5m2_decode(c) for c in range(0x7C)], dtype=np.float64)


def nearest_e5m2(y: np.ndarray, nan_sign_from: np.ndarray | None = None) -> np.ndarray:
    """Nearest finite e5m2 code (ties to the even code, sign kept, NaN ->
    0x7F | sign, infinities to the largest finite)."""
    return _nearest(y, TABLE_E5M2, nan_sign_from)


def nearest_e4m3fn(y: np.ndarray, nan_sign_from: np.ndarray | None = None) -> np.ndarray:
    """Nearest finite e4m3fn code to each fp32 value; on a tie the code whose
    lowest bit is 0; sign kept (so values that round to zero give +-0);
    NaN -> 0x7F with the sign of ``nan_sign_from`` (default: of y)."""
    return _nearest(y, TABLE, nan_sign_from)


def _nearest(y, table, nan_sign_from):
    y = np.asarray(y, dtype=np.float32).ravel()
    out = np.empty(y.size, dtype=np.uint8)
    sign = np.signbit(y)
    if nan_sign_from is not None:
        nsrc = np.signbit(np.asarray(nan_sign_from, dtype=np.float32).ravel())
    else:
        nsrc = sign
    with np.errstate(invalid="ignore"):
        a = np.abs(y.astype(np.float64))
    isnan = np.isnan(y)
    isinf = np.isinf(y)
    step = 1 << 15
    for s in range(0, y.size, step):
        aa = a[s:s + step].copy()
        bad = isnan[s:s + step] | isinf[s:s + step]
        aa[bad] = 0.0
        # Every table value is <= its largest entry, so for any |y| above
        # twice that the order of the distances is the same as at twice it;
        # clamping keeps the float64 differences exact (no cancellation).
        aa = np.minimum(aa, 2.0 * table[-1])
        d = np.abs(aa[:, None] - table[None, :])
        lo = np.argmin(d, axis=1)
        dmin = d[np.arange(lo.size), lo]
        nxt = np.minimum(lo + 1, table.size - 1)
        tie = (lo + 1 < table.size) & (d[np.arange(lo.size), nxt] == dmin)
        code = np.where(tie & (lo % 2 == 1), lo + 1, lo)
        code = np.where(isinf[s:s + step], table.size - 1, code)
        out[s:s + step] = code.astype(np.uint8)
    out = np.where(sign, out | 0x80, out).astype(np.uint8)
    out = np.where(isnan, np.where(nsrc, 0xFF, 0x7F), out).astype(np.uint8)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 patterns -> fp32 via torch's own bfloat16 dtype."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float32).numpy()


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def src_bits_to_f32(bits: np.ndarray, src_dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(bits) if src_dtype == "bf16" else f16_bits_to_f32(bits)


def scaled(bits: np.ndarray, src_dtype: str, inv_bits) -> tuple:
    """(x, y): decoded inputs and their fp32 product with the inverse scale."""
    x = src_bits_to_f32(bits, src_dtype)
    if inv_bits is None:
        return x, x.copy()
    inv = np.array([inv_bits], dtype=np.uint32).view(np.float32)[0]
    with np.errstate(all="ignore"):
        y = (x * np.float32(inv)).astype(np.float32)
    return x, y


def expected_codes(bits: np.ndarray, src_dtype: str, inv_bits, fmt: str = "e4m3fn") -> np.ndarray:
    x, y = scaled(bits, src_dtype, inv_bits)
    # an invalid product (inf * 0) is the negative default NaN
    bad = np.isnan(y) & ~np.isnan(x)
    y = y.copy()
    y[bad] = np.array([0xFFC00000], dtype=np.uint32).view(np.float32)[0]
    src = np.where(bad, y, x)
    f = nearest_e5m2 if fmt == "e5m2" else nearest_e4m3fn
    return f(y, nan_sign_from=src).reshape(np.shape(bits))


# ---------------------------------------------------------------------------
# Brute-force stores on tiny inputs (pure Python loops over tokens)
# ---------------------------------------------------------------------------

def copy_bruteforce(k_bytes, v_bytes, indices, row_bytes, k_stride, v_stride,
                    slots_total, cache_row, size_limit):
    """Python-level scatter copy into fresh sentinel caches.  Returns
    (k_cache, v_cache, bad_tokens)."""
    kc = bytearray(b"\xff" * (slots_total * cache_row))
    vc = bytearray(b"\xff" * (slots_total * cache_row))
    kb = bytes(k_bytes)
    vb = bytes(v_bytes)
    bad = []
    for t, loc in enumerate(int(i) for i in indices):
        if not (0 <= loc < size_limit):
            bad.append(t)
            continue
        kc[loc * cache_row: loc * cache_row + row_bytes] = kb[t * k_stride: t * k_stride + row_bytes]
        vc[loc * cache_row: loc * cache_row + row_bytes] = vb[t * v_stride: t * v_stride + row_bytes]
    return (np.frombuffer(bytes(kc), dtype=np.uint8).reshape(slots_total, cache_row),
            np.frombuffer(bytes(vc), dtype=np.uint8).reshape(slots_total, cache_row), bad)


# ---------------------------------------------------------------------------
# Dynamic scales: independent float32 reference
# ---------------------------------------------------------------------------

def dynamic_expected(bits: np.ndarray, src_dtype: str, num_heads: int, head_dim: int,
                     per_head: bool):
    """Per token row (bits [T, H*D]): group amax (NaN ignored) -> scale =
    max(amax / 448, 2^-126) (float32) -> inv = 1 / scale (float32) -> nearest
    e4m3fn of x * inv.  Returns (codes [T, H*D] uint8, scales [T, G] float32)."""
    T = bits.shape[0]
    x = src_bits_to_f32(bits[:, :num_heads * head_dim], src_dtype).reshape(T, num_heads, head_dim)
    G = num_heads if per_head else 1
    xg = x.reshape(T, G, -1)
    with np.errstate(all="ignore"):
        amax = np.fmax.reduce(np.abs(xg), axis=2, initial=np.float32(0.0)).astype(np.float32)
        scale = (amax / np.float32(448.0)).astype(np.float32)
        scale = np.maximum(scale, np.float32(2.0 ** -126)).astype(np.float32)
        inv = (np.float32(1.0) / scale).astype(np.float32)
        y = (xg * inv[:, :, None]).astype(np.float32)
    # an invalid product (inf * 0) is the negative default NaN
    bad = np.isnan(y) & ~np.isnan(xg)
    y[bad] = np.array([0xFFC00000], dtype=np.uint32).view(np.float32)[0]
    codes = nearest_e4m3fn(y.reshape(T, -1), nan_sign_from=np.where(bad, y, xg).reshape(T, -1))
    return codes.reshape(T, -1), scale
