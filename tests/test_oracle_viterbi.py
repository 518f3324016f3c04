"""Pins of the max-sum (Viterbi) trace oracle (``oracle.viterbi``).

Brute force over all K^L paths fixes the value and the tie rule; closed forms
fix the degenerate cases.  Each pin targets a plausible mistake: a dropped
edge, an off-by-one in the edge index, a transposed score matrix, a wrong
tie rule, a backtrack that reads the wrong table row.
"""

import itertools

import numpy as np
import pytest

from oracle import dflash as O
from oracle import viterbi as V


def _lattice(rng, L, K, integer=False):
    if integer:
        S = rng.integers(-3, 4, size=(L, K, K)).astype(np.float64)
    else:
        S = rng.standard_normal((L, K, K))
    S[0] = S[0, 0][None, :]  # edge 1 starts at the verified token: equal rows
    return S


def _brute(S):
    L, K, _ = S.shape
    best, arg = -np.inf, []
    for p in itertools.product(range(K), repeat=L):
        v = V.path_value(S, p)
        if v > best:
            best, arg = v, [p]
        elif v == best:
            arg.append(p)
    # smallest in reverse lexicographic order: compare j_L first
    return best, min(arg, key=lambda p: tuple(reversed(p)))


@pytest.mark.parametrize("L,K", [(1, 4), (2, 3), (3, 4), (4, 3), (4, 4), (5, 2)])
def test_brute_force_value_and_path(L, K):
    rng = np.random.default_rng([L, K, 1])
    for _ in range(20):
        S = _lattice(rng, L, K)
        cand = rng.integers(0, 1000, size=(L, K))
        path, draft, val, _ = V.viterbi_stream(S, cand)
        best, p = _brute(S)
        assert val == pytest.approx(best, abs=1e-12)
        assert tuple(path) == p
        np.testing.assert_array_equal(draft, cand[np.arange(L), path])


@pytest.mark.parametrize("L,K", [(2, 3), (3, 3), (4, 2), (3, 4)])
def test_brute_force_tie_rule_on_integer_scores(L, K):
    rng = np.random.default_rng([L, K, 2])
    for _ in range(40):
        S = _lattice(rng, L, K, integer=True)
        path, _, val, _ = V.viterbi_stream(S, np.zeros((L, K), np.int64))
        best, p = _brute(S)
        assert val == best
        assert tuple(path) == p


def test_predecessor_free_scores_give_independent_top1():
    # S[t, i, j] = U_t(j) for every i (zero embeddings): the max-sum path is
    # the per-position first argmax, the same as the greedy trace
    rng = np.random.default_rng(3)
    L, K = 6, 16
    U = rng.standard_normal((L, K))
    U[2, 5] = U[2, 1] = U[2].max() + 1.0  # a tie: the lower rank wins
    S = np.repeat(U[:, None, :], K, axis=1)
    path, _, val, _ = V.viterbi_stream(S, np.zeros((L, K), np.int64))
    np.testing.assert_array_equal(path, [O.argmax_first(U[t]) for t in range(L)])
    assert path[2] == 1
    assert val == pytest.approx(U.max(axis=1).sum(), abs=1e-12)
    gpath, _, _, _ = O.trace_stream(S, np.zeros((L, K), np.int64), 0.0, 0, 0)
    np.testing.assert_array_equal(path, gpath)


def test_one_position_is_the_row_argmax():
    S = np.array([[[0.5, 2.0, 2.0, -1.0]] * 4])
    path, _, val, _ = V.viterbi_stream(S, np.arange(4)[None, :])
    assert list(path) == [1] and val == 2.0


def test_hand_built_lattice_where_greedy_and_max_sum_differ():
    # edge 1: rank 0 worth 5, rank 1 worth 4; edge 2: only 1 -> 1 pays (10)
    S = np.zeros((2, 2, 2))
    S[0] = [[5.0, 4.0], [5.0, 4.0]]
    S[1] = [[0.0, 0.0], [0.0, 10.0]]
    path, _, val, _ = V.viterbi_stream(S, np.array([[7, 8], [9, 10]]))
    assert list(path) == [1, 1] and val == 14.0
    gpath, _, _, _ = O.trace_stream(S, np.zeros((2, 2), np.int64), 0.0, 0, 0)
    assert list(gpath) == [0, 0]                    # greedy takes 5 then 0
    assert V.path_value(S, gpath) == 5.0


def test_transposed_edge_matrix_is_caught():
    # predecessor rows vs candidate columns: only (row 1, col 0) of edge 2 pays
    S = np.zeros((2, 2, 2))
    S[0] = [[0.0, 1.0], [0.0, 1.0]]
    S[1] = [[0.0, 0.0], [3.0, 0.0]]
    path, _, val, _ = V.viterbi_stream(S, np.zeros((2, 2), np.int64))
    assert list(path) == [1, 0] and val == 4.0


def test_edge_constants_do_not_move_the_path_and_max_sum_beats_greedy():
    rng = np.random.default_rng(4)
    L, K = 7, 16
    for _ in range(10):
        S = _lattice(rng, L, K)
        path, _, val, _ = V.viterbi_stream(S, np.zeros((L, K), np.int64))
        c = rng.standard_normal(L)
        path2, _, val2, _ = V.viterbi_stream(S + c[:, None, None], np.zeros((L, K), np.int64))
        np.testing.assert_array_equal(path, path2)
        assert val2 == pytest.approx(val + c.sum(), abs=1e-9)
        gpath, _, _, _ = O.trace_stream(S, np.zeros((L, K), np.int64), 0.0, 0, 0)
        assert V.path_value(S, gpath) <= val + 1e-12
        assert V.path_value(S, path) == pytest.approx(val, abs=1e-12)


def test_margins_report_the_decisions_taken():
    S = np.zeros((2, 2, 2))
    S[0] = [[5.0, 4.0], [5.0, 4.0]]
    S[1] = [[0.0, 0.0], [0.0, 10.0]]
    _, _, _, m = V.viterbi_stream(S, np.zeros((2, 2), np.int64))
    # final choice: 14 vs 5 (gap 9); backtrack at edge 2 into rank 1: 14 vs 5
    assert [g for _, g, _ in m] == [9.0, 9.0]
