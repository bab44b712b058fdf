"""bench.py's output contract: the one JSON line, its fields and their
consistency; the multi-GPU refusal; the use of stored counter figures only
while they belong to the current kernel source."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import kvgen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_stored_traffic_is_dropped_for_another_source(monkeypatch):
    monkeypatch.setattr(bench, "source_sha", lambda: "0" * 64)
    assert bench.stored_traffic() is None


def test_stored_traffic_belongs_to_the_current_source():
    t = bench.stored_traffic()
    if t is None:
        pytest.skip("the counter summary was taken on another kernel source: the bench "
                    "reports traffic as null until the counters are taken again")
    b3 = kvgen.workload(3).algorithmic_bytes()
    b4 = kvgen.workload(4).algorithmic_bytes()
    # read and written bytes within a few percent of the algorithmic ones
    assert 0.98 < (t["copy_fetch_bytes"] + t["copy_write_bytes"]) / b3 < 1.05
    assert 0.98 < (t["fp8_fetch_bytes"] + t["fp8_write_bytes"]) / b4 < 1.05


def test_stored_traffic_absent_summary(monkeypatch, tmp_path):
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(tmp_path / "missing.md"))
    assert bench.stored_traffic() is None


@pytest.mark.gpu
def test_bench_line_contract():
    print("[gpu-case] bench.py --steps 3 --warmup 1 --no-decode --no-next --cpu-reps 1", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--no-decode", "--no-next", "--cpu-reps", "1"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                     ("steps", int), ("warmup", int), ("ms_per_step", float),
                     ("higher_is_better", bool), ("scaling", str), ("dtype", str),
                     ("data", str), ("config", dict), ("roofline", dict),
                     ("cpu_baseline", dict)):
        assert isinstance(d[key], typ), key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["scaling"] in ("weak", "strong")
    assert d["vs_baseline"] is None
    assert "workload" in d["config"] and "model" not in d["config"]
    b3 = kvgen.workload(3).algorithmic_bytes()
    b4 = kvgen.workload(4).algorithmic_bytes()
    assert d["config"]["bytes_per_step"] == b3 + b4
    # value is the step's bytes over the step time
    assert abs(d["value"] - (b3 + b4) / (d["ms_per_step"] * 1e-3) / 1e9) / d["value"] < 0.01
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["algorithmic_bytes"] == b3
    assert abs(rf["achieved"] - b3 / (rf["avg_launch_us"] * 1e-6) / 1e9) / rf["achieved"] < 0.01
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert 0.0 < rf["frac"] < 1.0
    assert rf["traffic"] is None or 0.98 < rf["traffic"] / b3 < 1.05
    # the bound fractions come with the secondary measurements (skipped here)
    assert rf["frac_of_serial_bound"] is None and rf["frac_of_destination_bound"] is None
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["sample"]
    assert "host_cpu_model" in cb and cb["host_cpus"] >= 1


def test_plain_reference_library_exports():
    import ctypes
    path = os.path.join(ROOT, "bench_plain.so")
    if not os.path.exists(path):
        pytest.skip("bench_plain.so not built")
    lib = ctypes.CDLL(path)
    for name in ("bench_plain_copy", "bench_plain_copy_chunks", "bench_plain_read2_write1",
                 "bench_plain_read", "bench_plain_write", "bench_plain_scatter_write",
                 "bench_plain_scatter_write_i64"):
        assert hasattr(lib, name), name
    vp, i64, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32
    lib.bench_plain_copy.argtypes = [vp, vp, i64, vp]
    lib.bench_plain_copy_chunks.argtypes = [vp, vp, i64, ctypes.c_int, vp]
    lib.bench_plain_read2_write1.argtypes = [vp, vp, i64, vp]
    lib.bench_plain_read.argtypes = [vp, vp, i64, u32, vp]
    lib.bench_plain_write.argtypes = [vp, i64, u32, vp]
    # argument errors return before any launch (no GPU needed)
    for chunks in (0, 1, 3, 16):
        assert lib.bench_plain_copy_chunks(16, 32, 16, chunks, None) == -1
    assert lib.bench_plain_copy_chunks(None, 32, 16, 2, None) == -1
    assert lib.bench_plain_copy_chunks(16, 32, 24, 8, None) == -1
    assert lib.bench_plain_copy_chunks(8, 32, 16, 4, None) == -1
    assert lib.bench_plain_copy(None, None, 16, None) == -1
    assert lib.bench_plain_copy(16, 32, 15, None) == -1
    assert lib.bench_plain_copy(8, 32, 16, None) == -1
    assert lib.bench_plain_read2_write1(16, 32, 0, None) == -1
    assert lib.bench_plain_read(None, 32, 16, 0, None) == -1
    assert lib.bench_plain_read(16, None, 16, 0, None) == -1
    assert lib.bench_plain_read(16, 32, 24, 0, None) == -1
    assert lib.bench_plain_read(8, 32, 16, 0, None) == -1
    assert lib.bench_plain_write(None, 16, 0, None) == -1
    assert lib.bench_plain_write(16, 0, 0, None) == -1
    assert lib.bench_plain_write(24, 16, 0, None) == -1
    for name in ("bench_plain_scatter_write", "bench_plain_scatter_write_i64"):
        sw = getattr(lib, name)
        sw.argtypes = [vp, vp, vp, i64, i64, i64, i64, u32, ctypes.c_int, vp]
        assert sw(None, 32, 64, 1, 2048, 2048, 8, 0, 0, None) == -1      # null cache
        assert sw(16, 32, 64, 0, 2048, 2048, 8, 0, 0, None) == -1        # no tokens
        for row in (0, 8, 1000, 4112):
            assert sw(16, 32, 64, 1, row, 4112, 8, 0, 0, None) == -1     # row not 16..4096 by 16
        assert sw(16, 32, 64, 1, 2048, 1024, 8, 0, 0, None) == -1        # stride below the row
        assert sw(16, 32, 64, 1, 2048, 2056, 8, 0, 0, None) == -1        # stride not 16-byte
        assert sw(16, 32, 66, 1, 2048, 2048, 8, 0, 0, None) == -1        # misaligned indices
        assert sw(16, 32, 64, 1, 2048, 2048, 0, 0, 0, None) == -1        # no slots
        for cap in (-2, 1, 3, 66):
            assert sw(16, 32, 64, 1, 2048, 2048, 8, 0, cap, None) == -1  # residency cap
    assert lib.bench_plain_scatter_write_i64(16, 32, 68, 1, 2048, 2048, 8, 0, 0, None) == -1


@pytest.mark.gpu
def test_plain_reference_kernels_move_the_right_bytes():
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "bench_plain.so"))
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.bench_plain_copy.argtypes = [vp, vp, i64, vp]
    lib.bench_plain_copy_chunks.argtypes = [vp, vp, i64, ctypes.c_int, vp]
    lib.bench_plain_read2_write1.argtypes = [vp, vp, i64, vp]
    dev = torch.device("cuda:0")
    sh = torch.cuda.current_stream().cuda_stream
    g = torch.Generator().manual_seed(5)
    for nbytes in (16, 4096, 4112, 1 << 20, (1 << 20) + 4080):
        print(f"[gpu-case] plain copy {nbytes} B", flush=True)
        src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).to(dev)
        dst = torch.zeros(nbytes + 4096, dtype=torch.uint8, device=dev)
        assert lib.bench_plain_copy(src.data_ptr(), dst.data_ptr(), nbytes, sh) == 0
        torch.cuda.synchronize()
        assert torch.equal(dst[:nbytes], src) and int(dst[nbytes:].sum()) == 0
        for chunks in (2, 4, 8):
            print(f"[gpu-case] plain copy {nbytes} B, {chunks} KiB per wave", flush=True)
            dst.zero_()
            assert lib.bench_plain_copy_chunks(src.data_ptr(), dst.data_ptr(), nbytes, chunks,
                                               sh) == 0
            torch.cuda.synchronize()
            assert torch.equal(dst[:nbytes], src) and int(dst[nbytes:].sum()) == 0
    lib.bench_plain_read.argtypes = [vp, vp, i64, ctypes.c_uint32, vp]
    lib.bench_plain_write.argtypes = [vp, i64, ctypes.c_uint32, vp]
    for nbytes in (16, 4096, 4112, (1 << 20) + 4080):
        print(f"[gpu-case] plain write / read {nbytes} B", flush=True)
        dst = torch.zeros(nbytes + 4096, dtype=torch.uint8, device=dev)
        assert lib.bench_plain_write(dst.data_ptr(), nbytes, 0x5A5A5A5A, sh) == 0
        torch.cuda.synchronize()
        words = dst[:nbytes].view(torch.int32).view(-1, 4).cpu().numpy().view(np.uint32)
        i = np.arange(nbytes // 16, dtype=np.uint64)
        h = ((i * 0x9E3779B1) & 0xFFFFFFFF).astype(np.uint32) ^ np.uint32(0x5A5A5A5A)
        want = np.stack([h, h ^ np.uint32(0x85EBCA6B), h ^ np.uint32(0xC2B2AE35),
                         h + np.uint32(0x27D4EB2F)], axis=1)
        np.testing.assert_array_equal(words, want)
        assert int(dst[nbytes:].sum()) == 0
        # the read-only kernel writes its sink only when a wave's XOR equals magic
        sink = torch.zeros(1024, dtype=torch.uint8, device=dev)
        assert lib.bench_plain_read(dst.data_ptr(), sink.data_ptr(), nbytes, 0x9E3779B9, sh) == 0
        torch.cuda.synchronize()
        assert int(sink.sum()) == 0
    for name in ("bench_plain_scatter_write", "bench_plain_scatter_write_i64"):
        getattr(lib, name).argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int64,
                                       ctypes.c_uint32, ctypes.c_int, vp]
    for T, row, cap, i64_idx in ((1, 1024, 0, False), (37, 2048, 12, False),
                                 (500, 3072, 0, False), (64, 4096, 12, False),
                                 (300, 1152, 0, True), (45, 16, 12, True), (70, 1008, 0, False)):
        print(f"[gpu-case] plain scatter write {T} rows of {row} B, cap {cap}, "
              f"int{64 if i64_idx else 32} indices", flush=True)
        slots, stride = 700, row + 64
        perm = np.random.default_rng(T).permutation(slots)[:T]
        idx = torch.from_numpy(perm.astype(np.int64 if i64_idx else np.int32))
        idx[0] = slots                               # out of range: skipped
        kc = torch.zeros(slots * stride, dtype=torch.uint8, device=dev)
        vc = torch.zeros_like(kc)
        fn = lib.bench_plain_scatter_write_i64 if i64_idx else lib.bench_plain_scatter_write
        assert fn(kc.data_ptr(), vc.data_ptr(), idx.to(dev).data_ptr(), T, row, stride, slots, 7,
                  cap, sh) == 0
        torch.cuda.synchronize()
        for cache, salt in ((kc, 7), (vc, 7 ^ 0x5BD1E995)):
            got = cache.view(slots, stride).cpu().numpy()
            want = np.zeros((slots, stride), dtype=np.uint8)
            lanes = np.arange(row // 16, dtype=np.uint64)        # 16-byte word c*64 + lane
            for t in range(1, T):
                h = ((t * 0x9E3779B1 + lanes) & 0xFFFFFFFF).astype(np.uint32) ^ np.uint32(salt)
                w = np.stack([h, h ^ np.uint32(0x85EBCA6B), h ^ np.uint32(0xC2B2AE35),
                              h + np.uint32(0x27D4EB2F)], axis=1)
                want[int(idx[t]), :row] = w.view(np.uint8).reshape(-1)
            np.testing.assert_array_equal(got, want)
    for waves in (1, 2, 3, 1001):
        print(f"[gpu-case] plain read2/write1 {waves} waves", flush=True)
        src = torch.randint(0, 256, (waves, 2, 1024), dtype=torch.uint8, generator=g).to(dev)
        dst = torch.zeros(waves + 4, 1024, dtype=torch.uint8, device=dev)
        assert lib.bench_plain_read2_write1(src.data_ptr(), dst.data_ptr(), waves, sh) == 0
        torch.cuda.synchronize()
        # lane l XORs bytes [16l, 16l + 16) of the two halves and stores the
        # first 8 bytes at 8l, the last 8 at 512 + 8l
        x = (src[:, 0] ^ src[:, 1]).view(waves, 64, 2, 8)
        want = torch.cat([x[:, :, 0].reshape(waves, 512), x[:, :, 1].reshape(waves, 512)], dim=1)
        assert torch.equal(dst[:waves], want) and int(dst[waves:].sum()) == 0
