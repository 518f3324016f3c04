"""The library's fp64 exponential (``exp_nonpos`` in csrc/device_util.hpp)
run on the host against the C library's exp.

Every fp64 accept test, trace weight and residual weight of the GPU path goes
through this function, so its stated bound (relative error below 1e-14 over
[-708, 0]) is checked here on the CPU: the header is compiled host-only with
hipcc (no device code, no GPU call) into a small filter program that maps
hexadecimal doubles on stdin to e^x on stdout.
"""

import math
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_draft_select_amd", "csrc")

PROGRAM = r"""
#include "device_util.hpp"
#include <cstdio>
int main() {
  double x;
  while (std::scanf("%la", &x) == 1) std::printf("%a\n", dfk::exp_nonpos(x));
  return 0;
}
"""


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def exp_host(tmp_path_factory):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("exp_nonpos")
    src, exe = d / "exp_host.cpp", d / "exp_host"
    src.write_text(PROGRAM)
    subprocess.run([cc, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17", "-I", CSRC,
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True,
                   capture_output=True)

    def run(xs):
        text = "\n".join(float(x).hex() for x in xs) + "\n"
        out = subprocess.run([str(exe)], input=text, capture_output=True, text=True, check=True).stdout
        return np.array([float.fromhex(v) for v in out.split()])
    return run


def _grid():
    rng = np.random.default_rng(11)
    ln2 = math.log(2.0)
    pts = [0.0, -0.0, -1e-300, -1e-17, -1e-9, -ln2 / 2, -ln2 / 2 - 1e-16, -ln2 / 2 + 1e-16, -ln2, -1.0,
           -10.0, -100.0, -700.0, -708.0]
    # arguments near every reduction boundary (n + 1/2) ln 2, where the
    # rounded n changes and |r| is largest
    pts += [-(n + 0.5) * ln2 + e for n in range(0, 1021, 7) for e in (-1e-12, 0.0, 1e-12)]
    pts += list(-rng.random(20000) * 708.0)
    pts += list(-rng.random(5000) * 2.0)
    pts += list(-np.exp(rng.uniform(-40, 0, 2000)))
    return np.array(pts, dtype=np.float64)


def test_relative_error_below_1e14_on_the_normal_range(exp_host):
    xs = _grid()
    got = exp_host(xs)
    ref = np.array([math.exp(x) for x in xs])
    rel = np.abs(got - ref) / ref
    assert rel.max() < 1e-14, (xs[rel.argmax()], rel.max())


def test_zero_and_underflow(exp_host):
    xs = np.array([0.0, -708.5, -720.0, -745.0, -746.0, -999.0, -1000.0, -1001.0, -1e6, -np.inf])
    got = exp_host(xs)
    assert got[0] == 1.0
    # past -708 the result leaves the normal range: it may lose relative
    # precision, but not absolute; far out it is exactly zero
    ref = np.array([math.exp(x) for x in xs])
    assert np.all(np.abs(got - ref) <= 1e-307)
    assert np.all(got[-4:] == 0.0)
    assert np.all(got >= 0.0)


def test_bound_catches_a_dropped_reduction_tail():
    # the same reduction written out in Python with the tail of ln 2 left
    # out: its error is far above the bound, so the bound is tight enough to
    # notice a mistake of that kind in the compiled code
    head = 0.693145751953125
    xs = _grid()[-3000:]
    n = np.rint(xs * 1.4426950408889634)
    r = xs - n * head
    bad = np.exp(r) * np.exp2(n)
    ref = np.exp(xs)
    assert (np.abs(bad - ref) / ref).max() > 1e-12
