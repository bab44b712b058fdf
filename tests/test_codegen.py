"""The store kernels' load order, read from the gfx950 code the compiler
makes of the library source (device-only assembly, no GPU needed).

Each wave must have all of its row loads in flight before it first waits
for one: written with loads under branches, the compiler can sink a load
into the branch of its store, or copy loaded registers where branches join,
and then waits for every load before issuing the next, one memory latency
after another (copies of 3 and 4 KiB rows ran 30% slower that way).  A
kernel that fails here has changed shape, not just timing.

Covered: every instantiation of the row copy, of the packed small-row copy,
of the FP8 store and of the dynamic-scale store (one pass or several, bf16
or fp16).  Left alone, the compiler issued only the first two loads of an
fp16 row of several passes before waiting on them (8192 tokens of 32x128
fp16 with per-token-head scales ran 9% slower than bf16 of the same size).
"""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "fp8_kv_quantization_amd"))
import _build  # noqa: E402

COVERED = (
    r"kvstore_copy_kernelILi\d+ELi\d+ELi\d+E[il]E",
    r"kvstore_copy_packed_kernelILi\d+E[il]E",
    r"kvstore_fp8_paged_kernelILi\d+ELb[01]ELb[01]ELb[01]E[il]E",
    r"kvstore_fp8_dynamic_kernelILi\d+ELb[01]ELb[01]ELb[01]E[il]E",
)


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(_build.HIPCC):
        pytest.skip("hipcc not found")
    out = str(tmp_path_factory.mktemp("asm") / "kvstore.s")
    flags = [f for f in _build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [_build.HIPCC, *flags, "--cuda-device-only", "-S", "-I",
           os.path.join(ROOT, "include"), _build.SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read().splitlines()


def kernels(lines):
    """{mangled name: instruction lines} for every store kernel."""
    out = {}
    for i, ln in enumerate(lines):
        m = re.match(r"^(_ZN\w*kvstore_(?:copy|fp8)\w*):", ln)
        if not m:
            continue
        body = []
        for ln2 in lines[i + 1:]:
            if ln2.startswith(".Lfunc_end"):
                break
            t = ln2.strip()
            if t and not t.startswith((";", ".")):
                body.append(t)
        out[m.group(1)] = body
    return out


def loads_before_first_wait(body):
    """(row loads issued before the first wait on vector memory, all row loads)."""
    loads = [n for n, t in enumerate(body) if t.startswith(("global_load", "buffer_load"))]
    waits = [n for n, t in enumerate(body) if t.startswith("s_waitcnt") and "vmcnt" in t]
    first_wait = waits[0] if waits else len(body)
    return sum(1 for n in loads if n < first_wait), len(loads)


def test_every_row_load_is_in_flight_before_the_first_wait(asm):
    ks = kernels(asm)
    covered = {k: b for k, b in ks.items() if any(re.search(p, k) for p in COVERED)}
    # 3 lane widths x (4 chunk counts + 2 with several tokens per wave) x 2
    # index types; packed: 3 lane widths x 2 index types; FP8: 1 or 2 passes
    # x 16 forms; dynamic: 1, 2 or 4 passes x 16 forms
    assert len(covered) == 36 + 6 + 32 + 48, sorted(covered)
    bad = {}
    for name, body in covered.items():
        before, total = loads_before_first_wait(body)
        assert total >= 1, name
        if before != total:
            bad[name] = (before, total)
    assert not bad, f"row loads issued after a wait: {bad}"


def test_the_index_load_is_issued_with_the_row_loads(asm):
    """The scalar index loads of the copy come after its row loads (so the
    row loads do not wait for them) and before its first wait (so the
    latencies overlap)."""
    ks = kernels(asm)
    for name, body in ks.items():
        if not re.search(COVERED[0], name):
            continue
        loads = [n for n, t in enumerate(body) if t.startswith("global_load")]
        first_wait = next(n for n, t in enumerate(body) if t.startswith("s_waitcnt") and "vmcnt" in t)
        idx = [n for n, t in enumerate(body) if re.match(r"s_load_dword(x2)? s\[?\d", t)
               and t.endswith(", 0x0") and "s[0:1]" not in t]
        assert idx, name
        assert loads[-1] < idx[0] < first_wait, (name, loads, idx, first_wait)
