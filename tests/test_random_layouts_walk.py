"""CPU bounds walk of every seeded random layout of the GPU parity test.

The oracle, built with AddressSanitizer, runs each layout over host buffers
of exactly the byte lengths the GPU test allocates on the device
(tests/_random_layouts.py): an access outside them would abort the walk.
The library addresses the same layout the same way, so a clean walk shows
that the device buffers hold every access of the GPU runs.  A planted short
cache shows that the walk does catch an overrun.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from tests import _random_layouts as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def asan_oracle(tmp_path_factory):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime for gcc")
    lib = str(tmp_path_factory.mktemp("asan") / "liboracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address",
                    "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-shared", "-fPIC",
                    oracle.SRC, "-o", lib, "-lm"], check=True)
    return rt, lib


def _walk(asan_oracle, body):
    rt, lib = asan_oracle
    script = (f"import sys\nsys.path.insert(0, {ROOT!r})\n"
              "import oracle\n"
              f"oracle._lib = oracle.load({lib!r})\n"
              "from tests import _random_layouts as R\n" + body)
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    return subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True,
                          timeout=900)


def test_every_random_layout_stays_inside_buffers_of_the_device_sizes(asan_oracle):
    r = _walk(asan_oracle, "for seed in R.SEEDS:\n"
                           "    op, L = R.draw(seed)\n"
                           "    R.run_oracle(op, L)\n"
                           "print('walked', len(R.SEEDS))\n")
    assert r.returncode == 0, r.stderr[-3000:]
    assert f"walked {len(R.SEEDS)}" in r.stdout


def test_the_walk_catches_a_short_cache(asan_oracle):
    op, L = R.draw(0)
    assert op == "copy"
    idx = L["idx"].astype(np.int64)
    top = int(idx[(idx >= 0) & (idx < L["limit"])].max())
    # the highest written slot ends half a row past the shortened cache
    short = L["off"] + top * L["row"] + L["row"] // 2
    r = _walk(asan_oracle, "op, L = R.draw(0)\n"
                           f"L['cache_bytes'] = {short}\n"
                           "R.run_oracle(op, L)\n"
                           "print('no overrun seen')\n")
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stdout + r.stderr[-2000:]
