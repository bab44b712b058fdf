"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of oracle/kvstore_oracle.c with one plausible slip
(a dropped term, a wrong sign rule, a wrong index or stride, an off-by-one),
built with gcc into a temporary directory and run through a fast subset of the
pins in a child process.  The real oracle passes that subset; every mutant
must fail it.  The oracle source itself is never modified.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "ties_away_from_zero": ("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    "ties_toward_zero": ("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl;"),
    "truncating_round": ("if (frac > 0.5) return fl + 1.0;", "if (frac > 0.99) return fl + 1.0;"),
    "overflow_to_nan": ("if (a > 448.0) return (uint8_t)(0x7E | s);",
                        "if (a > 448.0) return (uint8_t)(0x7F | s);"),
    "saturate_late": ("if (a > 448.0) return (uint8_t)(0x7E | s);",
                      "if (a > 480.0) return (uint8_t)(0x7E | s);"),
    "sign_by_compare": ("uint8_t s = signbit(y) ? 0x80 : 0x00;", "uint8_t s = (y < 0) ? 0x80 : 0x00;"),
    "subnormal_scale": ("round_half_even(a * 512.0)", "round_half_even(a * 256.0)"),
    "exponent_off_by_one": ("int e = ex - 1;", "int e = ex;"),
    "no_mantissa_carry": ("if (m == 16.0) {", "if (m == 17.0) {"),
    "dropped_scale": ("double p = (double)x * (double)inv;", "double p = (double)x;"),
    "fp16_bias": ("ldexp((double)(1024 + m), e - 25)", "ldexp((double)(1024 + m), e - 24)"),
    "fp16_subnormal": ("ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    "bf16_shift": ("(uint32_t)b << 16", "(uint32_t)b << 15"),
    "page_offset_swapped": ("cache[page * s_page + off * s_off + h * s_chead + d]",
                            "cache[off * s_page + page * s_off + h * s_chead + d]"),
    "head_stride_ignored": ("src + t * s_tok + h * s_head + 2 * d",
                            "src + t * s_tok + h * 2 * head_dim + 2 * d"),
    "bound_off_by_one": ("if (loc < 0 || loc >= size_limit) {", "if (loc < 0 || loc > size_limit) {"),
    "input_stride_ignored": ("k + t * k_stride", "k + t * row_bytes"),
    "index_stride_ignored": ("read_index(indices, idx_is_i64, t * idx_stride)",
                             "read_index(indices, idx_is_i64, t)"),
    "first_bad_keeps_max": ("t < *first_bad", "t > *first_bad"),
    "e5m2_overflow_to_inf": ("if (a > 57344.0) return (uint8_t)(0x7B | s);",
                             "if (a > 57344.0) return (uint8_t)(0x7C | s);"),
    "e5m2_subnormal_scale": ("round_half_even(a * 65536.0)", "round_half_even(a * 32768.0)"),
    "e5m2_bias": ("((e + 15) << 2)", "((e + 16) << 2)"),
    "e5m2_no_carry": ("if (m == 8.0) {", "if (m == 9.0) {"),
    "dyn_no_scale_floor": ("if (scale < FLT_MIN) scale = FLT_MIN;", ""),
    "dyn_inverse_in_one_step": ("float inv = 1.0f / scale;", "float inv = 448.0f / amax;"),
    "dyn_signed_amax": ("float a = fabsf(src_to_float(bits, src_is_fp16));",
                        "float a = src_to_float(bits, src_is_fp16);"),
    "dyn_wrong_fp8_max": ("float scale = amax / 448.0f;", "float scale = amax / 480.0f;"),
    "dyn_scale_page_offset_swapped": ("scales + page * sc_page + off * sc_off + g * sc_head",
                                      "scales + off * sc_page + page * sc_off + g * sc_head"),
    # V borrowing one of K's layout parameters
    "copy_v_uses_k_stride": ("v + t * v_stride", "v + t * k_stride"),
    "fp8_v_uses_k_input_strides": ("store_fp8_row(v, v_stride_token, v_stride_head,",
                                   "store_fp8_row(v, k_stride_token, k_stride_head,"),
    "fp8_vcache_uses_k_layout": ("vc_stride_offset, vc_stride_head, page, off",
                                 "kc_stride_offset, kc_stride_head, page, off"),
    "dyn_v_uses_k_input_stride": ("int64_t s_tok = x ? v_stride_token : k_stride_token;",
                                  "int64_t s_tok = k_stride_token;"),
    "dyn_v_uses_k_cache_layout": ("int64_t c_off = x ? vc_stride_offset : kc_stride_offset;",
                                  "int64_t c_off = kc_stride_offset;"),
    "dyn_v_uses_k_scale_layout": ("int64_t sc_head = x ? vs_stride_head : ks_stride_head;",
                                  "int64_t sc_head = ks_stride_head;"),
    "fp8_v_uses_k_inverse_scale": ("src_is_fp16, iv, fmt);", "src_is_fp16, ik, fmt);"),
}


def _run_battery(lib_path):
    env = dict(os.environ, PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-m", "tests._battery", lib_path], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    return r.returncode, (r.stdout + r.stderr)[-400:]


def test_unmutated_oracle_passes_battery():
    rc, out = _run_battery(oracle.build())
    assert rc == 0, out


def test_every_mutant_is_caught(tmp_path):
    src = open(oracle.SRC).read()
    libs = {}
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) >= 1, f"mutation site for {name} not found"
        path_c = tmp_path / f"{name}.c"
        path_c.write_text(src.replace(old, new))
        lib = str(tmp_path / f"lib{name}.so")
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-std=c11", "-shared", "-fPIC",
                        str(path_c), "-o", lib, "-lm"], check=True)
        libs[name] = lib
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = dict(zip(libs, ex.map(_run_battery, libs.values())))
    survived = [n for n, (rc, _) in results.items() if rc == 0]
    assert not survived, f"mutants not caught by the pins: {survived}"
