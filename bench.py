"""Benchmark of the KV-cache store on one MI355X.

One step = the whole store path once: a scatter copy of the prefill workload
(32768 tokens, 8 heads x 128 dims bf16, int32 indices into 2^21 slots of
16-slot pages) followed by a fused FP8 e4m3fn paged store (16384 tokens,
8 x 128 bf16, inverse scales 1/2.5 and 1/1.7, page 64, 2^21 slots).

Inputs are seeded synthetic data, resident in HBM before timing starts.  Calls
rotate over disjoint input/index sets (more than the 256 MB last-level
cache), so the figure is an HBM figure, not a cache figure.  The metric is
effective bandwidth: algorithmic bytes (K/V rows read + indices read + cache
rows written, + the two fp32 scales) per second.

Prints one JSON line.  ``--gpus N`` with N > 1 exits with a message: the
benchmark measures one GPU (the store needs no exchange between GPUs, so each
GPU of a larger job runs this same step on its own share).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
KERNEL_SRC = os.path.join(ROOT, "fp8_kv_quantization_amd", "csrc", "kvstore.hip")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_traffic_prefill_copy_fp8_paged.md")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=8, help="disjoint input/index sets rotated over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=21,
                    help="oracle runs of one full step (about 0.55 s each on one core)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also launch a plain device copy of this size (counter calibration)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-next", action="store_true", help="skip the next-row measurements")
    ap.add_argument("--copy-patterns", action="store_true",
                    help="only time the prefill copy over four destination patterns (12 launches "
                         "each: 2 untimed, 10 timed; for counter runs) and print that as the line")
    ap.add_argument("--copy-extents", action="store_true",
                    help="only time the prefill copy with its 16-slot runs drawn from cache "
                         "extents of 64 MiB .. 4 GiB per tensor (12 launches each, for counter "
                         "runs, then --extent-windows timed windows) and print that as the line")
    ap.add_argument("--extent-windows", type=int, default=3,
                    help="timed 50-call windows per extent after the 12 launches (0: none)")
    return ap.parse_args()


def source_sha() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()


def stored_traffic():
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    vals = dict(re.findall(r"^(\w+)\s*=\s*(\S+)\s*$", text, re.M))
    if vals.get("kernel_source_sha256") != source_sha():
        return None
    try:
        out = {k: float(vals[k]) for k in ("copy_fetch_bytes", "copy_write_bytes",
                                           "fp8_fetch_bytes", "fp8_write_bytes")}
    except KeyError:
        return None
    for k in ("wide_fetch_bytes", "wide_write_bytes", "tp_fetch_bytes", "tp_write_bytes"):
        if k in vals:
            out[k] = float(vals[k])
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported; the store shards with no exchange, so each GPU would run this "
              "same one-GPU step on its own share", file=sys.stderr)
        sys.exit(2)

    import torch

    import fp8_kv_quantization_amd as kv
    import kvgen

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S = args.sets

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    log("generating inputs")
    c3 = kvgen.workload(3)
    c4 = kvgen.workload(4)
    idx3 = kvgen.disjoint_index_sets(c3, S)      # set 0 = the workload's own indices
    idx4 = kvgen.disjoint_index_sets(c4, S)
    assert len(np.unique(np.concatenate(idx3))) == S * c3.num_tokens
    assert len(np.unique(np.concatenate(idx4))) == S * c4.num_tokens

    # Rotation sets: distinct device buffers; set s holds set 0's rows rolled
    # by s*997 tokens (same values, different memory).
    k3 = [to_dev(c3.k)]
    v3 = [to_dev(c3.v)]
    k4 = [to_dev(c4.k)]
    v4 = [to_dev(c4.v)]
    for s in range(1, S):
        k3.append(torch.roll(k3[0], s * 997, 0).contiguous())
        v3.append(torch.roll(v3[0], s * 997, 0).contiguous())
        k4.append(torch.roll(k4[0], s * 997, 0).contiguous())
        v4.append(torch.roll(v4[0], s * 997, 0).contiguous())
    i3 = [to_dev(a) for a in idx3]
    i4 = [to_dev(a) for a in idx4]
    inv_k = to_dev(np.array([c4.inv_k_bits], dtype=np.uint32).view(np.float32))
    inv_v = to_dev(np.array([c4.inv_v_bits], dtype=np.uint32).view(np.float32))

    R3 = c3.row_bytes
    kc3 = torch.full((c3.slots, R3), 0xFF, dtype=torch.uint8, device=dev)
    vc3 = torch.full_like(kc3, 0xFF)
    H, D, P = c4.num_heads, c4.head_dim, c4.page_size
    R4 = H * D
    kc4 = torch.full((c4.slots, R4), 0xFF, dtype=torch.uint8, device=dev)
    vc4 = torch.full_like(kc4, 0xFF)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def copy_call(s):
        st = kv.kvstore_copy(k3[s].data_ptr(), v3[s].data_ptr(), kc3.data_ptr(), vc3.data_ptr(),
                             i3[s].data_ptr(), kv.IDX_I32, 1, R3, c3.in_stride_bytes,
                             c3.in_stride_bytes, R3, c3.num_tokens, c3.slots, sh)
        if st:
            raise kv.KVStoreError(st, "kvstore_copy")

    def fp8_call(s):
        st = kv.kvstore_fp8_paged(
            k4[s].data_ptr(), v4[s].data_ptr(), kc4.data_ptr(), vc4.data_ptr(), i4[s].data_ptr(),
            kv.IDX_I32, 1, kv.SRC_BF16, H, D, c4.in_stride_bytes, 2 * D, c4.in_stride_bytes, 2 * D,
            P * R4, R4, D, P * R4, R4, D, c4.num_tokens, c4.slots, P, inv_k.data_ptr(),
            inv_v.data_ptr(), sh)
        if st:
            raise kv.KVStoreError(st, "kvstore_fp8_paged")

    if args.copy_patterns:
        out = {"metric": "prefill copy launch time by destination pattern", "unit": "us",
               "higher_is_better": False, "n_gpus": 1, "data": "synthetic",
               "config": {"workload": "prefill copy (32768 tok, 8x128 bf16, int32, 2^21 slots), "
                                      "index sets replaced per pattern", "rotation_sets": S},
               "patterns": bench_patterns(kv, torch, kvgen, c3, k3, v3, kc3, vc3, S, sh,
                                          windows=1, n=10, warm=2)}
        print(json.dumps(out), flush=True)
        return

    if args.copy_extents:
        named = {f"{mib}MiB": kvgen.extent_index_sets(c3, mib << 20, S) for mib in kvgen.EXTENT_MIB}
        sample = bench_index_sets(kv, torch, c3, k3, v3, kc3, vc3, S, sh, named,
                                  windows=1, n=10, warm=2)
        out = {"metric": "prefill copy launch time by the extent its 16-slot runs are drawn from",
               "unit": "us", "higher_is_better": False, "n_gpus": 1, "data": "synthetic",
               "config": {"workload": "prefill copy (32768 tok, 8x128 bf16, int32, 2^21 slots), "
                                      "index sets replaced per extent", "rotation_sets": S},
               "counter_sample_12_launches": sample}
        if args.extent_windows > 0:
            out["extents"] = bench_index_sets(kv, torch, c3, k3, v3, kc3, vc3, S, sh, named,
                                              windows=args.extent_windows, n=50, warm=100)
        print(json.dumps(out), flush=True)
        return

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        log(f"calibration copy of {args.calib_copy_mib} MiB launched 3 times")

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        copy_call(i % S)
        fp8_call(i % S)
    torch.cuda.synchronize()

    # Timed region: K steps.  The K copy launches are issued back to back,
    # then the K FP8 launches (the two halves of a step share no data), with
    # one HIP event before, between and after, all on the launch stream, so
    # each kernel's average launch duration is measured without per-launch
    # event overhead.
    K = args.steps
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    log(f"timing {K} steps over {S} rotation sets")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        copy_call(i % S)
    e1.record(stream)
    for i in range(K):
        fp8_call(i % S)
    e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    copy_ms_total = e0.elapsed_time(e1)
    fp8_ms_total = e1.elapsed_time(e2)
    ms_per_step = max(e0.elapsed_time(e2), wall * 1e3) / K

    st, fb, bc = kv.kvstore_check_error(sh)
    if st != kv.OK:
        raise RuntimeError(f"device error flag set: first bad token {fb}, count {bc}")

    # Sampled parity on the timed buffers: set 0's slots hold set 0's rows.
    log("checking set-0 rows against the inputs")
    rows3 = kc3.index_select(0, i3[0].long())
    assert torch.equal(rows3, k3[0].view(torch.uint8).view(c3.num_tokens, -1)[:, :R3]), \
        "prefill copy: cache rows differ from input rows"

    b3 = c3.algorithmic_bytes()
    b4 = c4.algorithmic_bytes()
    copy_us = copy_ms_total * 1e3 / K
    fp8_us = fp8_ms_total * 1e3 / K
    value = (b3 + b4) / (ms_per_step * 1e-3) / 1e9

    hot = patterns = extents = alternating = None
    if not args.no_next:
        alternating = bench_alternating(torch, copy_call, fp8_call, b3 + b4, S)
        hot = bench_hot(torch, copy_call, fp8_call, b3, b4)
        patterns = bench_patterns(kv, torch, kvgen, c3, k3, v3, kc3, vc3, S, sh)
        extents = bench_index_sets(
            kv, torch, c3, k3, v3, kc3, vc3, S, sh,
            {f"{mib}MiB": kvgen.extent_index_sets(c3, mib << 20, S) for mib in kvgen.EXTENT_MIB})

    next_rows = None
    if not args.no_next:
        next_rows = bench_next_rows(kv, torch, c4, k4, v4, i4, S, sh)
        next_rows.update(bench_small_rows(kv, torch, c3, k3, v3, i3, S, sh))
        next_rows.update(bench_narrow_rows(kv, torch, c3, k3, v3, i3, S, sh))

    wide = bench_wide_strided(kv, torch, dev, kvgen, to_dev)
    traffic = stored_traffic()
    if traffic is not None and "wide_fetch_bytes" in traffic:
        wide["traffic"] = int(traffic["wide_fetch_bytes"] + traffic["wide_write_bytes"])
    if traffic is not None and "tp_fetch_bytes" in traffic and next_rows is not None:
        next_rows["copy_tp_share_256B_rows"]["traffic"] = int(traffic["tp_fetch_bytes"] +
                                                              traffic["tp_write_bytes"])
    plain = bound = None
    if not args.no_next:
        plain = bench_plain_kernels(torch, dev, b3, c4, S)
        bound = bench_serial_bound(
            torch, dev, c3, c4, copy_us, fp8_us,
            dest_sets={"prefill_copy": (kc3, vc3, i3, R3, c3.slots),
                       "fp8_paged": (kc4, vc4, i4, R4, c4.slots)})

    # Launch-bound decode-size figures last: the idle gaps of their
    # single-call latency loop leave the GPU slow to return to full speed for
    # the bandwidth-bound timings above.
    decode = tiny = fp8_decode = None
    if not args.no_decode:
        decode = bench_decode(kv, torch, dev, kvgen, to_dev, 2,
                              "decode copy (256 tok, 8x128 bf16, int64, 2^20 slots)")
        tiny = bench_decode(kv, torch, dev, kvgen, to_dev, 1,
                            "tiny copy (16 tok, 2x64 bf16, int32, 256 slots)")
        fp8_decode = bench_fp8_decode(kv, torch, dev, kvgen, to_dev)

    roofline = {
        "bound": "hbm",
        "kernel": "kvstore_copy_kernel<16, 2, 1, int> (prefill copy)",
        "achieved": round(b3 / (copy_us * 1e-6) / 1e9, 1),
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": round(b3 / (copy_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "traffic": None if traffic is None else int(traffic["copy_fetch_bytes"] + traffic["copy_write_bytes"]),
        "algorithmic_bytes": b3,
        "avg_launch_us": round(copy_us, 3),
        # the same launch against the same-run bounds of serial_bound: plain
        # read-only + write-only at 1 GiB, and read-only + write-only into the
        # copy's own destinations
        "frac_of_serial_bound": None if bound is None else
        bound["prefill_copy"]["frac_of_bound_asymptotic"],
        "frac_of_destination_bound": None if bound is None else
        bound["prefill_copy"].get("frac_of_bound_workload_destinations"),
    }
    breakdown = {
        "prefill_copy": {"avg_launch_us": round(copy_us, 3), "bytes": b3,
                         "GB/s": round(b3 / (copy_us * 1e-6) / 1e9, 1),
                         "frac_of_peak": round(b3 / (copy_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        "fp8_paged": {"avg_launch_us": round(fp8_us, 3), "bytes": b4,
                      "GB/s": round(b4 / (fp8_us * 1e-6) / 1e9, 1),
                      "frac_of_peak": round(b4 / (fp8_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                      "traffic": None if traffic is None else
                      int(traffic["fp8_fetch_bytes"] + traffic["fp8_write_bytes"])},
    }

    del k3, v3, k4, v4, kc3, vc3, kc4, vc4
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(c3, c4, args.cpu_reps)

    out = {
        "metric": "effective HBM GB/s (K/V+idx read + cache write)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic (seeded; inputs resident in HBM; rotated over disjoint sets)",
        "config": {
            "workload": "prefill copy (32768 tok, 8x128 bf16, int32, 2^21 slots, 16-slot pages) "
                        "+ fused FP8 e4m3fn paged store (16384 tok, 8x128 bf16, int32, "
                        "page 64, 2^21 slots, inv scales 1/2.5 1/1.7)",
            "bytes_per_step": b3 + b4,
            "rotation_sets": S,
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "breakdown": breakdown,
        "decode_copy": decode,
        "tiny_copy": tiny,
        "fp8_decode": fp8_decode,
        "wide_strided_copy": wide,
        "next_rows": next_rows,
        "plain_kernels_same_bytes": plain,
        "serial_bound": bound,
        "step_alternating": alternating,
        "copy_destination_patterns": patterns,
        "copy_destination_extents": extents,
        "hot_non_rotated": hot,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def time_calls(torch, call, S, n=50, reps=3, warm=500):
    """Median over `reps` windows of the average time of `n` back-to-back
    calls (rotating over S sets), after `warm` untimed calls; HIP events on
    the current stream.  Returns microseconds per call.  The long warm-up
    matters after the idle gaps of the single-call latency loop: with 20
    warm-up calls the conversion-heavy stores measured up to 7% slower."""
    stream = torch.cuda.current_stream()
    for i in range(warm):
        call(i % S)
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            call(i % S)
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / n)
    return statistics.median(out)


def bench_alternating(torch, copy_call, fp8_call, step_bytes, S, n=50, warm=20):
    """The step as a serving loop issues it: the copy and the FP8 store
    alternate, so whatever written state one kernel leaves behind is paid by
    the other inside the timed region (the headline times each kernel's
    launches back to back instead).  Median of three windows of n steps."""
    for i in range(warm):
        copy_call(i % S)
        fp8_call(i % S)
    torch.cuda.synchronize()
    r = []
    stream = torch.cuda.current_stream()
    for _ in range(3):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            copy_call(i % S)
            fp8_call(i % S)
        b.record(stream)
        torch.cuda.synchronize()
        r.append(a.elapsed_time(b) * 1e3 / n)
    us = statistics.median(r)
    return {"us_per_step": round(us, 3), "GB/s": round(step_bytes / (us * 1e-6) / 1e9, 1)}


def bench_hot(torch, copy_call, fp8_call, b3, b4, n=50):
    """The step's two kernels on one input/index set, the same every call
    (not rotated): the 256 MB last-level cache can serve part of the reads
    and absorb part of the writes, so these are not HBM figures; the
    headline figures are the rotated ones."""
    out = {"note": "set 0 every call, not rotated: the last-level cache (256 MB) may serve part "
                   "of each call; secondary figures, not HBM bandwidth"}
    for name, call, b in (("prefill_copy", copy_call, b3), ("fp8_paged", fp8_call, b4)):
        us = time_calls(torch, lambda s, call=call: call(0), 1, n=n, warm=100)
        out[name] = {"avg_launch_us": round(us, 3), "bytes": b,
                     "GB/s": round(b / (us * 1e-6) / 1e9, 1)}
    return out


def bench_patterns(kv, torch, kvgen, c3, k3, v3, kc3, vc3, S, sh, windows=3, n=50, warm=200):
    """The prefill copy (same rows, same library call) with its index sets
    replaced by four destination patterns (kvgen.pattern_index_sets):
    contiguous slots, 16-slot runs inside a 64 MiB extent, the workload's
    16-slot runs over the 4 GiB cache, single slots over the cache."""
    named = {pat: kvgen.pattern_index_sets(c3, pat, S) for pat in kvgen.DEST_PATTERNS}
    return bench_index_sets(kv, torch, c3, k3, v3, kc3, vc3, S, sh, named, windows, n, warm)


def bench_index_sets(kv, torch, c3, k3, v3, kc3, vc3, S, sh, named, windows=3, n=50, warm=200):
    """The prefill copy (same rows, same library call) with its index sets
    replaced by each entry of `named` (S host index arrays per name), in
    order.  Average launch time per entry (median of `windows` windows of n
    calls after `warm` calls, HIP events on the launch stream), rotated over
    the S sets."""
    import numpy as np
    R, T = c3.row_bytes, c3.num_tokens
    dev = k3[0].device
    out = {}
    for pat, sets in named.items():
        idx = [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in sets]

        def call(s):
            st = kv.kvstore_copy(k3[s].data_ptr(), v3[s].data_ptr(), kc3.data_ptr(), vc3.data_ptr(),
                                 idx[s].data_ptr(), kv.IDX_I32, 1, R, c3.in_stride_bytes,
                                 c3.in_stride_bytes, R, T, c3.slots, sh)
            if st:
                raise kv.KVStoreError(st, "kvstore_copy")

        us = time_calls(torch, call, S, n=n, reps=windows, warm=warm)
        b = c3.algorithmic_bytes()
        out[pat] = {"avg_launch_us": round(us, 3), "GB/s": round(b / (us * 1e-6) / 1e9, 1)}
        del idx
    st, _, _ = kv.kvstore_check_error(sh)
    assert st == kv.OK
    return out


def _random_bytes(torch, dev, n, seed):
    """n random bytes on the device: the plain kernels' sources (writing
    all-zero or constant lines measured faster than varied data on this GPU,
    so constant fills would flatter the ceilings)."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev, generator=g)


def _plain_lib():
    """bench_plain.so (built next to this file by __graft_entry__.build()),
    with its argument types set; None if it is not built."""
    import ctypes
    path = os.path.join(ROOT, "bench_plain.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    vp, i64, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32
    lib.bench_plain_copy.argtypes = [vp, vp, i64, vp]
    lib.bench_plain_copy_chunks.argtypes = [vp, vp, i64, ctypes.c_int, vp]
    lib.bench_plain_read2_write1.argtypes = [vp, vp, i64, vp]
    lib.bench_plain_read.argtypes = [vp, vp, i64, u32, vp]
    lib.bench_plain_write.argtypes = [vp, i64, u32, vp]
    for name in ("bench_plain_scatter_write", "bench_plain_scatter_write_i64"):
        getattr(lib, name).argtypes = [vp, vp, vp, i64, i64, i64, i64, u32, ctypes.c_int, vp]
    return lib


PLAIN_COPY_KIB_PER_WAVE = (2, 4, 8)


def plain_copy_us(torch, dev, nbytes, S, n=50):
    """Average launch time of the fastest hand-written plain contiguous copy
    moving nbytes in all (half read, half written), rotated over S buffer
    pairs: the copy with 2, 4 and 8 KiB per wave is timed and the fastest
    kept (small copies run faster with more bytes per wave).  Returns
    (us, KiB per wave), or (None, None) if bench_plain.so is not built."""
    lib = _plain_lib()
    if lib is None:
        return None, None
    half = nbytes // 2 // 16 * 16
    sh = torch.cuda.current_stream().cuda_stream
    src = [_random_bytes(torch, dev, half, 100 + s) for s in range(S)]
    dst = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(S)]
    best = (None, None)
    for kib in PLAIN_COPY_KIB_PER_WAVE:
        def copy(s, kib=kib):
            if lib.bench_plain_copy_chunks(src[s].data_ptr(), dst[s].data_ptr(), half, kib,
                                           sh) != 0:
                raise RuntimeError("bench_plain_copy_chunks failed")

        us = time_calls(torch, copy, S, n=n)
        if best[0] is None or us < best[0]:
            best = (us, kib)
    del src, dst
    torch.cuda.empty_cache()
    return best


def plain_read_us(torch, dev, lib, sink, nbytes, S, n=50):
    """Average time of the plain read-only kernel over `nbytes` (rounded up
    to 16), rotating over S buffers of random bytes."""
    sh = torch.cuda.current_stream().cuda_stream
    nbytes = (nbytes + 15) // 16 * 16
    bufs = [_random_bytes(torch, dev, nbytes, 200 + s) for s in range(S)]

    def call(s):
        if lib.bench_plain_read(bufs[s].data_ptr(), sink.data_ptr(), nbytes, 0x9E3779B9, sh):
            raise RuntimeError("bench_plain_read failed")

    us = time_calls(torch, call, S, n=n)
    del bufs
    torch.cuda.empty_cache()
    return us


def bench_serial_bound(torch, dev, c3, c4, copy_us, fp8_us, dest_sets=None, n=50):
    """Same-run attainable bound for the step's two kernels.  HBM serves a
    kernel's read and write streams one after the other, so a kernel that
    reads r bytes and writes w bytes takes at least r/R + w/W, with R and W
    the read-only and write-only rates of plain streaming kernels
    (bench_plain.hip, each in the fastest form measured).  Two forms: R and W
    measured at the kernel's own byte counts (each plain launch pays its own
    launch ramp, so this bound is the looser one) and at 1 GiB per launch
    (near the asymptotic rates).  With `dest_sets` ({kernel: (k_cache,
    v_cache, S device index arrays, row bytes, slots)}; caches whose slot
    row is `row bytes` long at a stride of `row bytes`), each kernel also
    gets the bound of its own destinations: the read-only time plus a
    write-only kernel that writes its rows to the same slots (no reads)."""
    lib = _plain_lib()
    if lib is None:
        return None
    sh = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(1024, dtype=torch.uint8, device=dev)

    def read_us(nbytes, S):
        return plain_read_us(torch, dev, lib, sink, nbytes, S, n)

    def write_us(nbytes, S):
        nbytes = (nbytes + 15) // 16 * 16
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(S)]

        def call(s):
            if lib.bench_plain_write(bufs[s].data_ptr(), nbytes, s, sh):
                raise RuntimeError("bench_plain_write failed")

        us = time_calls(torch, call, S, n=n)
        del bufs
        torch.cuda.empty_cache()
        return us

    gib = 1 << 30
    r_inf = gib / (read_us(gib, 3) * 1e-6) / 1e9
    w_inf = gib / (write_us(gib, 3) * 1e-6) / 1e9
    out = {"method": "bound = read-only time of r bytes + write-only time of w bytes (plain "
                     "streaming kernels of bench_plain.hip: non-temporal loads, one wave per 2 KiB; "
                     "sc1 16-byte stores, one wave per 4 KiB; rotated buffers of random bytes); "
                     "at_size: both plain launches at the kernel's own byte counts; "
                     "asymptotic: rates of 1 GiB launches",
           "read_GBs_1GiB": round(r_inf, 1), "write_GBs_1GiB": round(w_inf, 1)}
    T3, T4 = c3.num_tokens, c4.num_tokens
    rows = (("prefill_copy", copy_us, 2 * T3 * c3.row_bytes + T3 * c3.indices.itemsize,
             2 * T3 * c3.row_bytes, 8),
            ("fp8_paged", fp8_us, 2 * T4 * 2 * c4.row_elems + T4 * c4.indices.itemsize + 8,
             2 * T4 * c4.row_elems, 16))
    for name, k_us, r, w, S in rows:
        tr, tw = read_us(r, S), write_us(w, S)
        b_inf = (r / r_inf + w / w_inf) * 1e-3
        out[name] = {"read_bytes": r, "write_bytes": w, "kernel_us": round(k_us, 3),
                     "read_only_us": round(tr, 3), "write_only_us": round(tw, 3),
                     "bound_us_at_size": round(tr + tw, 3),
                     "frac_of_bound_at_size": round((tr + tw) / k_us, 4),
                     "bound_us_asymptotic": round(b_inf, 3),
                     "frac_of_bound_asymptotic": round(b_inf / k_us, 4)}
    if dest_sets is not None:
        def scatter_us(kc, vc, sets, T, R, slots, cap):
            def call(s):
                if lib.bench_plain_scatter_write(kc.data_ptr(), vc.data_ptr(), sets[s].data_ptr(),
                                                 T, R, R, slots, s, cap, sh):
                    raise RuntimeError("bench_plain_scatter_write failed")
            return time_calls(torch, call, len(sets), n=n)

        for name, (kc, vc, idx, R, slots) in dest_sets.items():
            k_us = out[name]["kernel_us"]
            T = int(idx[0].numel())
            # fastest of uncapped and of 12 waves per CU (the copy's residency)
            wl = min(scatter_us(kc, vc, idx, T, R, slots, cap) for cap in (0, 12))
            cont = [torch.arange(s * T, (s + 1) * T, dtype=torch.int32, device=dev)
                    for s in range(len(idx))]
            ct = min(scatter_us(kc, vc, cont, T, R, slots, cap) for cap in (0, 12))
            tr = out[name]["read_only_us"]
            out[name].update({
                "write_only_contiguous_slots_us": round(ct, 3),
                "write_only_workload_destinations_us": round(wl, 3),
                "bound_us_workload_destinations": round(tr + wl, 3),
                "frac_of_bound_workload_destinations": round((tr + wl) / k_us, 4)})
        out["workload_destinations"] = (
            "write-only kernel (bench_plain_scatter_write): the kernel's rows (K and V) written "
            "to its own index sets' slots with no reads, 16-byte sc1 stores, the faster of "
            "uncapped and 12 waves per CU; and the same into contiguous slots")
    return out


def bench_plain_kernels(torch, dev, copy_bytes, c4, S, n=50):
    """Same-GPU reference points for the two kernels of the step: torch's own
    device copy moving the prefill copy's byte count (contiguous, no index,
    no scatter), torch's own bf16 -> float8_e4m3fn cast over the FP8
    workload's element count (contiguous in and out, no scale, no paging),
    and the hand-written plain kernels of bench_plain.hip, each rotated over
    S buffer sets like the step."""
    out = {}
    half = copy_bytes // 2
    src = [_random_bytes(torch, dev, half, 400 + s) for s in range(S)]
    dst = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(S)]
    us = time_calls(torch, lambda s: dst[s].copy_(src[s]), S, n=n)
    out["torch_copy"] = {"bytes": 2 * half, "avg_launch_us": round(us, 3),
                         "GB/s": round(2 * half / (us * 1e-6) / 1e9, 1),
                         "frac_of_peak": round(2 * half / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    del src, dst
    elems = 2 * c4.num_tokens * c4.num_heads * c4.head_dim
    try:
        src = [torch.randn(elems, device=dev).to(torch.bfloat16) for _ in range(S)]
        dst = [torch.empty(elems, dtype=torch.float8_e4m3fn, device=dev) for _ in range(S)]
        us = time_calls(torch, lambda s: dst[s].copy_(src[s]), S, n=n)
        nbytes = 3 * elems
        out["torch_cast_bf16_to_e4m3fn"] = {
            "bytes": nbytes, "avg_launch_us": round(us, 3),
            "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        del src, dst
    except (RuntimeError, TypeError) as e:   # cast not available in this torch build
        out["torch_cast_bf16_to_e4m3fn"] = {"error": str(e)[:200]}
    torch.cuda.empty_cache()
    out.update(bench_hand_plain(torch, dev, copy_bytes, elems, S, n))
    return out


def bench_hand_plain(torch, dev, copy_bytes, fp8_elems, S, n=50):
    """The hand-written plain kernels of bench_plain.hip (built next to this
    file by __graft_entry__.build()): a contiguous copy of the prefill copy's
    byte count, and the FP8 store's per-wave shape (2 KiB read, 1 KiB
    written) over its wave count, with no index, scatter or conversion.
    Empty if the library is not built."""
    lib = _plain_lib()
    if lib is None:
        return {}
    sh = torch.cuda.current_stream().cuda_stream
    out = {}
    half = copy_bytes // 2 // 16 * 16
    us, kib = plain_copy_us(torch, dev, 2 * half, S, n)
    out["hand_plain_copy"] = {"bytes": 2 * half, "avg_launch_us": round(us, 3),
                              "kib_per_wave": kib,
                              "GB/s": round(2 * half / (us * 1e-6) / 1e9, 1),
                              "frac_of_peak": round(2 * half / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    waves = fp8_elems // 1024                   # one wave per 1024 elements (2 KiB of bf16)
    src = [_random_bytes(torch, dev, waves * 2048, 300 + s) for s in range(S)]
    dst = [torch.empty(waves * 1024, dtype=torch.uint8, device=dev) for _ in range(S)]

    def shape(s):
        if lib.bench_plain_read2_write1(src[s].data_ptr(), dst[s].data_ptr(), waves, sh) != 0:
            raise RuntimeError("bench_plain_read2_write1 failed")

    us = time_calls(torch, shape, S, n=n)
    nbytes = waves * 3072
    out["hand_plain_read2k_write1k"] = {"bytes": nbytes, "waves": waves,
                                        "avg_launch_us": round(us, 3),
                                        "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                                        "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    del src, dst
    torch.cuda.empty_cache()
    return out


def bench_next_rows(kv, torch, c4, k4, v4, i4, S, sh, n=50):
    """The fused FP8 store with scales computed in the kernel (per token and
    per token-head) on the FP8 workload's inputs, rotated like the main step."""
    H, D, P = c4.num_heads, c4.head_dim, c4.page_size
    R = H * D
    dev = k4[0].device
    kc = torch.full((c4.slots, R), 0xFF, dtype=torch.uint8, device=dev)
    vc = torch.full_like(kc, 0xFF)
    out = {}
    for per_head in (False, True):
        G = H if per_head else 1
        ks = torch.zeros((c4.slots, G), dtype=torch.float32, device=dev)
        vs = torch.zeros_like(ks)

        def call(s):
            st = kv.kvstore_fp8_paged_dynamic(
                k4[s].data_ptr(), v4[s].data_ptr(), kc.data_ptr(), vc.data_ptr(), i4[s].data_ptr(),
                kv.IDX_I32, 1, kv.SRC_BF16, H, D, c4.in_stride_bytes, 2 * D, c4.in_stride_bytes,
                2 * D, P * R, R, D, P * R, R, D, ks.data_ptr(), vs.data_ptr(),
                kv.SCALE_PER_TOKEN_HEAD if per_head else kv.SCALE_PER_TOKEN,
                P * G * 4, G * 4, 4 if per_head else 0, P * G * 4, G * 4, 4 if per_head else 0,
                c4.num_tokens, c4.slots, P, sh)
            if st:
                raise kv.KVStoreError(st, "kvstore_fp8_paged_dynamic")

        us = time_calls(torch, call, S, n)
        T = c4.num_tokens
        b = 2 * T * 2 * R + T * 4 + 2 * T * R + 2 * T * G * 4
        out["fp8_dynamic_" + ("per_head" if per_head else "per_token")] = {
            "workload": "fused FP8 paged store, scales computed per "
                        + ("token and head" if per_head else "token")
                        + " (16384 tok, 8x128 bf16, int32, page 64)",
            "avg_launch_us": round(us, 3), "bytes": b, "GB/s": round(b / (us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        del ks, vs
    # the same store into e5m2 caches, given scales
    ik = torch.tensor([0.4], dtype=torch.float32, device=dev)
    iv = torch.tensor([1.0 / 1.7], dtype=torch.float32, device=dev)

    def call_e5m2(s):
        st = kv.kvstore_fp8_paged_e5m2(
            k4[s].data_ptr(), v4[s].data_ptr(), kc.data_ptr(), vc.data_ptr(), i4[s].data_ptr(),
            kv.IDX_I32, 1, kv.SRC_BF16, H, D, c4.in_stride_bytes, 2 * D, c4.in_stride_bytes,
            2 * D, P * R, R, D, P * R, R, D, c4.num_tokens, c4.slots, P, ik.data_ptr(),
            iv.data_ptr(), sh)
        if st:
            raise kv.KVStoreError(st, "kvstore_fp8_paged_e5m2")

    us = time_calls(torch, call_e5m2, S, n)
    b = c4.algorithmic_bytes()
    out["fp8_e5m2"] = {
        "workload": "fused FP8 paged store into e5m2 caches (16384 tok, 8x128 bf16, int32, "
                    "page 64, inv scales 1/2.5 1/1.7)",
        "avg_launch_us": round(us, 3), "bytes": b, "GB/s": round(b / (us * 1e-6) / 1e9, 1),
        "frac_of_peak": round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    st, _, _ = kv.kvstore_check_error(sh)
    assert st == kv.OK
    del kc, vc
    return out


def bench_small_rows(kv, torch, c3, k3, v3, i3, S, sh, n=100):
    """Tensor-parallel share of the prefill copy: one 128-dim bf16 head per
    GPU, i.e. 256-byte rows (packed four to a wave), same tokens and slots."""
    dev = k3[0].device
    R = 256
    ks = [k3[s][:, :128].contiguous() for s in range(S)]
    vs = [v3[s][:, :128].contiguous() for s in range(S)]
    kc = torch.full((c3.slots, R), 0xFF, dtype=torch.uint8, device=dev)
    vc = torch.full_like(kc, 0xFF)

    def call(s):
        st = kv.kvstore_copy(ks[s].data_ptr(), vs[s].data_ptr(), kc.data_ptr(), vc.data_ptr(),
                             i3[s].data_ptr(), kv.IDX_I32, 1, R, R, R, R, c3.num_tokens, c3.slots,
                             sh)
        if st:
            raise kv.KVStoreError(st, "kvstore_copy")

    us = time_calls(torch, call, S, n)
    T = c3.num_tokens
    b = 2 * T * R * 2 + T * 4
    st, _, _ = kv.kvstore_check_error(sh)
    assert st == kv.OK
    del kc, vc, ks, vs
    torch.cuda.empty_cache()
    plain, plain_kib = plain_copy_us(torch, dev, b, S, n)
    return {"copy_tp_share_256B_rows": {
        "workload": "prefill copy with one 128-dim bf16 head per GPU (32768 tok, 256 B rows, "
                    "int32, 2^21 slots in 16-slot pages)",
        "avg_launch_us": round(us, 3), "bytes": b, "GB/s": round(b / (us * 1e-6) / 1e9, 1),
        "frac_of_peak": round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "plain_copy_same_bytes_us": None if plain is None else round(plain, 3),
        "plain_copy_kib_per_wave": plain_kib,
        "frac_of_plain_copy": None if plain is None else round(plain / us, 4)}}


def bench_narrow_rows(kv, torch, c3, k3, v3, i3, S, sh, n=50):
    """Rows whose size is a multiple of 8 or 4 bytes but not of 16, which the
    copy moves with 8- or 4-byte lanes: the prefill copy's tokens and index
    sets, each row the first bytes of the token's 2 KiB row (input stride
    2 KiB), cache rows at a stride of their own size; beside each, the
    16-byte-lane row of the next multiple of 64 bytes in the same run."""
    dev = k3[0].device
    T = c3.num_tokens
    out = {}
    for R, name in ((1024, "copy_1024B_rows_16B_lanes"), (1000, "copy_1000B_rows_8B_lanes"),
                    (512, "copy_512B_rows_16B_lanes"), (500, "copy_500B_rows_4B_lanes")):
        kc = torch.full((c3.slots, R), 0xFF, dtype=torch.uint8, device=dev)
        vc = torch.full_like(kc, 0xFF)

        def call(s, kc=kc, vc=vc, R=R):
            st = kv.kvstore_copy(k3[s].data_ptr(), v3[s].data_ptr(), kc.data_ptr(), vc.data_ptr(),
                                 i3[s].data_ptr(), kv.IDX_I32, 1, R, c3.in_stride_bytes,
                                 c3.in_stride_bytes, R, T, c3.slots, sh)
            if st:
                raise kv.KVStoreError(st, "kvstore_copy")

        us = time_calls(torch, call, S, n)
        st, _, _ = kv.kvstore_check_error(sh)
        assert st == kv.OK
        # every stored row of set S - 1 (the last call) equals its input bytes
        ii = i3[(n - 1) % S].long()[:64]
        src = k3[(n - 1) % S].view(torch.uint8).view(T, -1)[:64, :R]
        assert torch.equal(kc.index_select(0, ii), src), name
        b = 2 * T * R * 2 + T * 4
        lanes = 16 if R % 16 == 0 else 8 if R % 8 == 0 else 4
        out[name] = {
            "workload": f"prefill copy's tokens and slots ({T} tok, int32, 2^21 slots in "
                        f"16-slot pages), {R} B rows, {lanes}-byte lanes",
            "avg_launch_us": round(us, 3), "bytes": b, "GB/s": round(b / (us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        del kc, vc
        torch.cuda.empty_cache()
    return {"copy_rows_off_16_bytes": out}


def bench_decode(kv, torch, dev, kvgen, to_dev, n_workload, label):
    """A launch-bound copy (workload 1: tiny copy, 2: decode copy): per-call
    time back to back, single-call latency, and per-call time when the calls
    are replayed from a captured HIP graph (how a serving loop issues them),
    all from HIP events, over 16 disjoint index sets."""
    c2 = kvgen.workload(n_workload)
    S = 16
    sets = kvgen.disjoint_index_sets(c2, S)
    k = to_dev(c2.k)
    v = to_dev(c2.v)
    idx = [to_dev(a) for a in sets]
    R = c2.row_bytes
    code = kv.IDX_I64 if c2.indices.dtype == np.int64 else kv.IDX_I32
    kc = torch.full((c2.slots, R), 0xFF, dtype=torch.uint8, device=dev)
    vc = torch.full_like(kc, 0xFF)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def call(s, on=None):
        st = kv.kvstore_copy(k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                             idx[s].data_ptr(), code, 1, R, c2.in_stride_bytes,
                             c2.in_stride_bytes, R, c2.num_tokens, c2.slots,
                             sh if on is None else on)
        if st:
            raise kv.KVStoreError(st, "kvstore_copy")

    for i in range(20):
        call(i % S)
    torch.cuda.synchronize()
    n = 400
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        call(i % S)
    e1.record(stream)
    torch.cuda.synchronize()
    b2b_us = e0.elapsed_time(e1) * 1e3 / n
    lat = []
    for i in range(200):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call(i % S)
        b.record(stream)
        b.synchronize()
        lat.append(a.elapsed_time(b) * 1e3)
    # one graph holding S calls (one per index set), replayed back to back
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(S):
            call(s, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    reps = 25
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / (reps * S)
    del g
    st, _, _ = kv.kvstore_check_error(sh)
    assert st == kv.OK
    del kc, vc
    return {"workload": label,
            "us_per_call_back_to_back": round(b2b_us, 3),
            "us_single_call_median": round(statistics.median(lat), 3),
            "us_per_call_graph_replay": round(graph_us, 3),
            "bytes": c2.algorithmic_bytes()}


def bench_fp8_decode(kv, torch, dev, kvgen, to_dev, T=256):
    """The fused FP8 paged store at decode size (256 tokens, 8x128 bf16,
    int32, page 64, 2^21 slots, inverse scales 1/2.5 and 1/1.7): per-call
    time back to back, single-call latency, and per call when 16 calls
    captured in one HIP graph are replayed, over 16 disjoint index sets."""
    c = kvgen.workload(4, tokens=T)
    S = 16
    sets = kvgen.disjoint_index_sets(c, S)
    k = to_dev(c.k)
    v = to_dev(c.v)
    idx = [to_dev(a) for a in sets]
    ik = to_dev(np.array([c.inv_k_bits], dtype=np.uint32).view(np.float32))
    iv = to_dev(np.array([c.inv_v_bits], dtype=np.uint32).view(np.float32))
    H, D, P = c.num_heads, c.head_dim, c.page_size
    R = H * D
    kc = torch.full((c.slots, R), 0xFF, dtype=torch.uint8, device=dev)
    vc = torch.full_like(kc, 0xFF)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def call(s, on=None):
        st = kv.kvstore_fp8_paged(k.data_ptr(), v.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                                  idx[s].data_ptr(), kv.IDX_I32, 1, kv.SRC_BF16, H, D,
                                  c.in_stride_bytes, 2 * D, c.in_stride_bytes, 2 * D, P * R, R, D,
                                  P * R, R, D, c.num_tokens, c.slots, P, ik.data_ptr(),
                                  iv.data_ptr(), sh if on is None else on)
        if st:
            raise kv.KVStoreError(st, "kvstore_fp8_paged")

    b2b_us = time_calls(torch, call, S, n=400, reps=1, warm=200)
    lat = []
    for i in range(200):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call(i % S)
        b.record(stream)
        b.synchronize()
        lat.append(a.elapsed_time(b) * 1e3)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(S):
            call(s, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for _ in range(20):
        g.replay()
    torch.cuda.synchronize()
    reps = 25
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / (reps * S)
    del g
    st, _, _ = kv.kvstore_check_error(sh)
    assert st == kv.OK
    del kc, vc
    return {"workload": "fused FP8 paged store at decode size (256 tok, 8x128 bf16, int32, "
                        "page 64, 2^21 slots)",
            "us_per_call_back_to_back": round(b2b_us, 3),
            "us_single_call_median": round(statistics.median(lat), 3),
            "us_per_call_graph_replay": round(graph_us, 3),
            "bytes": c.algorithmic_bytes()}


def bench_wide_strided(kv, torch, dev, kvgen, to_dev, S=16, n=50):
    """Wide strided copy (8192 tokens, 1x576 fp16 = 1152 B rows read at a
    1280 B row stride, int64, 2^19 slots): average launch time over S
    disjoint input/index sets (about 600 MB per cycle, above the last-level
    cache), median of three windows."""
    c5 = kvgen.workload(5)
    sets = kvgen.disjoint_index_sets(c5, S)
    k = [to_dev(c5.k)]
    v = [to_dev(c5.v)]
    for s in range(1, S):
        k.append(torch.roll(k[0], s * 997, 0).contiguous())
        v.append(torch.roll(v[0], s * 997, 0).contiguous())
    idx = [to_dev(a) for a in sets]
    R = c5.row_bytes
    kc = torch.full((c5.slots, R), 0xFF, dtype=torch.uint8, device=dev)
    vc = torch.full_like(kc, 0xFF)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def call(s):
        st = kv.kvstore_copy(k[s].data_ptr(), v[s].data_ptr(), kc.data_ptr(), vc.data_ptr(),
                             idx[s].data_ptr(), kv.IDX_I64, 1, R, c5.in_stride_bytes,
                             c5.in_stride_bytes, R, c5.num_tokens, c5.slots, sh)
        if st:
            raise kv.KVStoreError(st, "kvstore_copy")

    us = time_calls(torch, call, S, n)
    st, _, _ = kv.kvstore_check_error(sh)
    assert st == kv.OK
    b = c5.algorithmic_bytes()
    del k, v
    torch.cuda.empty_cache()
    # its two halves launched apart: plain read-only of its read bytes, and a
    # write-only kernel writing its rows to the same slots (no reads), the
    # faster of uncapped and 12 waves per CU.  At this launch size each half
    # pays its own launch ramp, so their sum is no bound on the copy.
    dest = None
    lib = _plain_lib()
    if lib is not None:
        T = c5.num_tokens
        sink = torch.zeros(1024, dtype=torch.uint8, device=dev)
        tr = plain_read_us(torch, dev, lib, sink, 2 * T * R + T * 8, S, n)

        def scatter(cap):
            def w(s):
                if lib.bench_plain_scatter_write_i64(kc.data_ptr(), vc.data_ptr(),
                                                     idx[s].data_ptr(), T, R, R, c5.slots, s,
                                                     cap, sh):
                    raise RuntimeError("bench_plain_scatter_write_i64 failed")
            return time_calls(torch, w, S, n)

        tw = min(scatter(cap) for cap in (0, 12))
        dest = {"read_only_us": round(tr, 3), "write_only_workload_destinations_us": round(tw, 3),
                "sum_us": round(tr + tw, 3), "kernel_over_sum": round(us / (tr + tw), 4)}
    del kc, vc
    torch.cuda.empty_cache()
    plain, plain_kib = plain_copy_us(torch, dev, b, S, n)
    return {"workload": "wide strided copy (8192 tok, 1x576 fp16, input row stride 640 elements, "
                        "int64, 2^19 slots)",
            "avg_launch_us": round(us, 3), "bytes": b, "GB/s": round(b / (us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "rotation_sets": S,
            "plain_copy_same_bytes_us": None if plain is None else round(plain, 3),
            "plain_copy_kib_per_wave": plain_kib,
            "frac_of_plain_copy": None if plain is None else round(plain / us, 4),
            "halves_launched_apart": dest}


def cpu_baseline(c3, c4, reps):
    """The CPU oracle (single thread) on the same step: set 0 of both
    workloads into full-size host caches."""
    import oracle
    lib = oracle.load()
    log("cpu baseline: allocating host caches")
    kc3 = np.full((c3.slots, c3.row_bytes), 0xFF, dtype=np.uint8)
    vc3 = np.full_like(kc3, 0xFF)
    kc4 = np.full((c4.slots, c4.row_elems), 0xFF, dtype=np.uint8)
    vc4 = np.full_like(kc4, 0xFF)
    times = []
    for r in range(reps):
        t0 = time.perf_counter()
        oracle.run_case(c3, kc3, vc3, lib=lib)
        oracle.run_case(c4, kc4, vc4, lib=lib)
        times.append(time.perf_counter() - t0)
        log(f"cpu baseline rep {r}: {times[-1]:.3f} s")
    t = statistics.median(times)
    b = c3.algorithmic_bytes() + c4.algorithmic_bytes()
    return {"value": round(b / t / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} runs of one full step (prefill copy 32768 tok + fused FP8 paged "
                      f"16384 tok, set 0) into full-size host caches, {sum(times):.1f} s of "
                      f"CPU work; median run",
            "seconds_per_step": round(t, 4),
            "host_cpus": os.cpu_count(), "host_cpu_model": host_cpu_model()}


def host_cpu_model():
    """The host CPU's model name from /proc/cpuinfo, or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
