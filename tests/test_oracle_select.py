"""Pins of the oracle's gate (S2), pair scores (S3) and trace (S4).

Pins: closed forms of the gate and of the score on structured embeddings;
check (1) zero bilinear weights reduce the selector to independent top-1
picks; check (4) brute-force enumeration of every lattice path at tiny K and
L (the greedy walk is the unique greedy-consistent path; at T > 0 the
enumerated path law sums to one and matches the sampled frequencies).
"""

import itertools
import math

import numpy as np
import pytest
from scipy import special, stats

import synth
from oracle import dflash


# ---------------------------------------------------------------- gate

def test_gate_zero_context_is_one_half():
    W = np.random.default_rng(0).standard_normal((32, 64))
    assert np.array_equal(dflash.gate(np.zeros(64), W), np.full(32, 0.5))


def test_gate_single_input_closed_form():
    # h = e_i selects column i of W: g = 1 / (1 + e^{-W[:, i]})
    W = np.linspace(-4, 4, 8 * 5).reshape(8, 5)
    h = np.zeros(5)
    h[3] = 1.0
    want = np.array([1.0 / (1.0 + math.exp(-w)) for w in W[:, 3]])
    assert np.allclose(dflash.gate(h, W), want, rtol=0, atol=1e-15)


def test_gate_is_monotone_and_symmetric():
    W = np.eye(4)
    h = np.array([-3.0, -1.0, 1.0, 3.0])
    g = dflash.gate(h, W)
    assert np.all(np.diff(g) > 0)
    assert abs(g[0] + g[3] - 1.0) < 1e-15 and abs(g[1] + g[2] - 1.0) < 1e-15


# ---------------------------------------------------------------- scores

def test_score_one_hot_embeddings():
    # one-hot embeddings: the bilinear term is g[k] when predecessor and
    # candidate share dimension k, else zero
    r, K = 6, 4
    g = np.array([0.1, 0.2, 0.3, 0.4, 0.5, 0.6])
    pred_dims = [0, 1, 2, 3]
    cand_dims = [3, 1, 5, 0]
    P = np.eye(r)[pred_dims]
    C = np.eye(r)[cand_dims]
    u = np.array([1.0, -2.0, 0.5, 3.0])
    S = dflash.pair_scores(P, C, u, g)
    for i in range(K):
        for j in range(K):
            want = u[j] + (g[pred_dims[i]] if pred_dims[i] == cand_dims[j] else 0.0)
            assert S[i, j] == want


def test_score_zero_embeddings_is_drafter_logit():
    u = np.array([3.0, 2.0, 2.0, -1.0])
    S = dflash.pair_scores(np.zeros((4, 8)), np.zeros((4, 8)), u, np.full(8, 0.7))
    assert np.array_equal(S, np.tile(u, (4, 1)))


def test_score_scalar_gate_is_scaled_dot_product():
    rng = np.random.default_rng(5)
    P, C = rng.standard_normal((3, 16)), rng.standard_normal((5, 16))
    u = rng.standard_normal(5)
    S = dflash.pair_scores(P, C, u, np.full(16, 0.25))
    for i in range(3):
        for j in range(5):
            assert abs(S[i, j] - (u[j] + 0.25 * sum(P[i, k] * C[j, k] for k in range(16)))) < 1e-12


# ---------------------------------------------------------------- check (1)

@pytest.mark.parametrize("ties", [False, True])
def test_zero_embeddings_give_independent_top1(ties):
    inp = synth.make(1, set_id=3, zero_E=True, ties=ties)
    out = dflash.cycle_stream(inp, 0)
    U = dflash.widen(inp["U"][0], "f32")
    assert np.all(out["path_rank"] == 0)
    for t in range(inp["L"]):
        assert out["draft_tok"][t] == int(np.argmax(U[t]))


def test_zero_embeddings_sampled_trace_is_drafter_softmax():
    # with E = 0 the score row is U_t over C_t, so q_t = softmax(U_t(C_t)/T)
    inp = synth.make(1, set_id=4, zero_E=True, T=0.7)
    out = dflash.cycle_stream(inp, 0)
    T = float(np.float32(0.7))
    for t in range(inp["L"]):
        want = special.softmax(out["cand_val"][t] / T)
        assert np.allclose(out["q"][t], want, rtol=1e-12, atol=0)


# ---------------------------------------------------------------- check (4)

def _random_lattice(rng, L, K):
    S = rng.standard_normal((L, K, K))
    S[0] = S[0][0][None, :]                       # edge 1: all rows equal
    cand = rng.permutation(50)[: L * K].reshape(L, K)
    return S, cand


@pytest.mark.parametrize("seed", range(30))
def test_greedy_trace_is_unique_greedy_consistent_path(seed):
    rng = np.random.default_rng(seed)
    L, K = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    S, cand = _random_lattice(rng, L, K)
    path, draft, q, _ = dflash.trace_stream(S, cand, 0.0, 1, 0)
    consistent = []
    for p in itertools.product(range(K), repeat=L):
        prev, ok = 0, True
        for t in range(L):
            if S[t, prev, p[t]] != S[t, prev].max():
                ok = False
                break
            prev = p[t]
        if ok:
            consistent.append(p)
    assert consistent == [tuple(path)]
    assert np.array_equal(draft, cand[np.arange(L), path])
    assert np.array_equal(q, np.eye(K)[path])


def test_greedy_trace_ties_take_lowest_rank():
    S = np.zeros((2, 3, 3))
    S[0] = [[1.0, 1.0, 0.5]] * 3
    S[1] = [[0.0, 0.0, 0.0], [2.0, 3.0, 3.0], [0.0, 0.0, 0.0]]
    path, _, _, _ = dflash.trace_stream(S, np.arange(6).reshape(2, 3), 0.0, 1, 0)
    assert list(path) == [0, 0]
    S[0] = [[1.0, 2.0, 2.0]] * 3
    path, _, _, _ = dflash.trace_stream(S, np.arange(6).reshape(2, 3), 0.0, 1, 0)
    assert list(path) == [1, 1]


def _path_law(S, T):
    L, K, _ = S.shape
    law = {}
    for p in itertools.product(range(K), repeat=L):
        prob, prev = 1.0, 0
        for t in range(L):
            prob *= special.softmax(S[t, prev] / T)[p[t]]
            prev = p[t]
        law[p] = prob
    return law


def test_sampled_trace_law_sums_to_one_and_q_matches():
    rng = np.random.default_rng(1)
    S, cand = _random_lattice(rng, 3, 3)
    law = _path_law(S, 0.8)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    path, _, q, _ = dflash.trace_stream(S, cand, 0.8, 99, 3)
    prev = 0
    for t in range(3):
        assert np.allclose(q[t], special.softmax(S[t, prev] / 0.8), rtol=1e-12, atol=0)
        prev = path[t]


def test_sampled_trace_frequencies_match_enumeration():
    rng = np.random.default_rng(2)
    L, K, T = 3, 3, 1.3
    S, cand = _random_lattice(rng, L, K)
    law = _path_law(S, T)
    paths = list(law)
    n = 6000
    counts = dict.fromkeys(paths, 0)
    for c in range(n):
        path, _, _, _ = dflash.trace_stream(S, cand, T, 0xABCDEF, c)
        counts[tuple(path)] += 1
    obs = np.array([counts[p] for p in paths], dtype=float)
    exp = np.array([law[p] for p in paths]) * n
    keep = exp >= 5
    obs_k = np.append(obs[keep], obs[~keep].sum())
    exp_k = np.append(exp[keep], exp[~keep].sum())
    if exp_k[-1] == 0:
        obs_k, exp_k = obs_k[:-1], exp_k[:-1]
    assert stats.chisquare(obs_k, exp_k).pvalue > 1e-4
