"""Pins of the oracle's top-K candidate extraction (S1).

Pins: brute force with Python's own sort on tiny rows, the argmax invariant,
exact tie and signed-zero handling, and the generator's planted ranks (a
property fixed by how the inputs were built, not by the oracle).
"""

import numpy as np
import pytest

import synth
from oracle import dflash


def _brute(row, K):
    order = sorted(range(len(row)), key=lambda i: (-float(row[i]), i))
    return order[:K]


@pytest.mark.parametrize("seed", range(20))
def test_matches_python_sort(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(1, 60))
    K = int(rng.integers(1, min(V, 16) + 1))
    row = np.round(rng.standard_normal(V) * 2) / 2          # many exact ties
    idx, val = dflash.topk_row(row, K)
    assert list(idx) == _brute(row, K)
    assert np.array_equal(val, row[idx])


def test_rank0_is_first_argmax():
    rng = np.random.default_rng(3)
    for _ in range(50):
        row = rng.integers(-3, 4, size=200).astype(np.float64)
        idx, _ = dflash.topk_row(row, 5)
        assert idx[0] == int(np.argmax(row))                 # numpy: first max


def test_signed_zero_ties_by_index():
    row = np.array([-1.0, 0.0, -0.0, 0.0, -0.0, -2.0])
    idx, val = dflash.topk_row(row, 4)
    assert list(idx) == [1, 2, 3, 4]
    row2 = np.array([-0.0, 0.0])
    assert list(dflash.topk_row(row2, 2)[0]) == [0, 1]


def test_all_equal_row_takes_lowest_indices():
    idx, _ = dflash.topk_row(np.full(1000, 1.5), 16)
    assert list(idx) == list(range(16))


def test_widen_bf16_is_exact():
    x = np.array([1.0, -2.5, 3.140625, 0.0, -0.0, 65280.0], dtype=np.float32)
    bits = synth.bf16_bits(x)
    assert np.array_equal(dflash.widen(bits, "bf16"), x.astype(np.float64))


def test_planted_ranks_are_recovered():
    # the generator plants token y at a drawn rank with a bf16 value strictly
    # between its neighbours: the oracle's top-16 must place it there
    inp = synth.make(3, set_id=9, B=4, V=4096)
    U = dflash.widen(inp["U"], "bf16")
    hits = 0
    for b in range(inp["B"]):
        for t in range(inp["L"]):
            idx, _ = dflash.topk_row(U[b, t], 16)
            y, rk = inp["planted"][b, t], inp["planted_rank"][b, t]
            if rk <= 16:
                assert idx[rk - 1] == y
                hits += 1
            else:
                assert y not in idx
    assert hits > 0
