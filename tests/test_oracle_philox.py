"""Pins of the oracle's Philox4x32-10 and uniform conversions.

Pins: the published known-answer vectors (tests/golden/philox4x32_10_kat.txt),
an independent library implementation (rocRAND's philox4x32_10 engine run on
the host), exact-representability of the uniforms, and a uniformity test.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kat_rows():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            v = [int(x, 16) for x in line.split()]
            rows.append((tuple(v[0:4]), tuple(v[4:6]), tuple(v[6:10])))
    return rows


@pytest.mark.parametrize("ctr,key,want", _kat_rows())
def test_kat_scalar(ctr, key, want):
    assert philox.philox4x32_10(key, ctr) == want


@pytest.mark.parametrize("ctr,key,want", _kat_rows())
def test_kat_vectorised(ctr, key, want):
    got = philox.philox4x32_10_np(key[0], key[1], *ctr)
    assert tuple(int(g) for g in got) == want


def test_vectorised_matches_scalar_on_random_counters():
    rng = np.random.default_rng(7)
    n = 200
    k = rng.integers(0, 2**32, size=(n, 2), dtype=np.uint64)
    c = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64)
    got = philox.philox4x32_10_np(k[:, 0], k[:, 1], c[:, 0], c[:, 1], c[:, 2], c[:, 3])
    for i in range(n):
        want = philox.philox4x32_10((k[i, 0], k[i, 1]), tuple(c[i]))
        assert tuple(int(g[i]) for g in got) == want


def test_against_rocrand_engine(tmp_path):
    """rocRAND's host-callable philox4x32_10 engine agrees word for word."""
    hipcc = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
    if hipcc is None or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    exe = tmp_path / "prref"
    subprocess.run([hipcc, "-O1", os.path.join(GOLDEN, "rocrand_philox_ref.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, cwd=str(tmp_path))
    rng = np.random.default_rng(11)
    cases = []
    for _ in range(64):
        seed = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        c0 = int(rng.integers(0, 2**32))
        c1 = int(rng.integers(0, 2**30))      # offset*4 must stay below 2^64
        c2 = int(rng.integers(0, 2**32))
        c3 = int(rng.integers(0, 2**32))
        cases.append((seed, c0, c1, c2, c3))
    cases.append((0, 0, 0, 1, 0))
    cases.append(((3 << 32) | 5, 17, 0, 8, 1))
    inp = "\n".join(" ".join(str(v) for v in c) for c in cases) + "\n"
    out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout
    lines = out.strip().splitlines()
    assert len(lines) == len(cases)
    for (seed, c0, c1, c2, c3), line in zip(cases, lines):
        want = tuple(int(x) for x in line.split())
        got = philox.philox4x32_10((seed & 0xFFFFFFFF, seed >> 32), (c0, c1, c2, c3))
        assert got == want


def test_stream_block_counter_layout():
    # key = seed halves, counter = (cycle lo, cycle hi, position, slot)
    seed, cycle = (7 << 32) | 9, (2 << 32) | 5
    assert philox.stream_block(seed, cycle, 3, 1) == philox.philox4x32_10((9, 7), (5, 2, 3, 1))


def test_u01_f32_exact_and_open_interval():
    for w in [0, 1, 511, 512, 0x7FFFFFFF, 0x80000000, 0xFFFFFFFE, 0xFFFFFFFF]:
        u = philox.u01_f32(w)
        assert 0.0 < u < 1.0
        assert float(np.float32(u)) == u
    assert philox.u01_f32(0) == 2.0 ** -24
    assert philox.u01_f32(0xFFFFFFFF) == 1.0 - 2.0 ** -24


def test_u01_f64_exact_and_open_interval():
    for hi, lo in [(0, 0), (0, 4095), (0, 4096), (0xFFFFFFFF, 0xFFFFFFFF), (0x80000000, 0)]:
        u = philox.u01_f64(hi, lo)
        assert 0.0 < u < 1.0
        k = (((hi << 32) | lo) >> 12)
        assert u == (2 * k + 1) * 2.0 ** -53
    assert philox.u01_f64(0xFFFFFFFF, 0xFFFFFFFF) == 1.0 - 2.0 ** -53


def test_uniformity_of_draws():
    words = philox.philox4x32_10_np(123, 456, np.arange(20000), 0, 3, 0)
    u = np.array([philox.u01_f32(int(w)) for w in words[1]])
    # Kolmogorov-Smirnov against U(0,1); a broken word order or a constant
    # stream fails by a wide margin
    assert stats.kstest(u, "uniform").pvalue > 1e-4
    counts = np.bincount((u * 16).astype(int), minlength=16)
    assert stats.chisquare(counts).pvalue > 1e-4


def test_distinct_counters_give_distinct_blocks():
    seen = set()
    for t in range(1, 18):
        for slot in (0, 1):
            for cyc in range(4):
                seen.add(philox.stream_block(5, cyc, t, slot))
    assert len(seen) == 17 * 2 * 4
