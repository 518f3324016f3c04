"""Pins of the oracle's verify (S5, S6).

Pins: check (2) at T = 0 the output equals an independent autoregressive
greedy decode of the target rows; check (3) chi-square tests at tiny vocab
that every emitted token, conditional on its position being reached, follows
the target distribution p; the closed-form acceptance probability
sum_b min(p(b), q(b)); q = p always accepts; the residual draw has the same
law for any chunk size; the degenerate-residual fallback samples p.
"""

import numpy as np
import pytest
from scipy import special, stats

import synth
from oracle import dflash


def _greedy_decode(Z, draft):
    """Autoregressive greedy reference written independently of the oracle."""
    L = len(draft)
    out = []
    for t in range(L + 1):
        best = sorted(range(Z.shape[1]), key=lambda i: (-Z[t, i], i))[0]
        out.append(best)
        if t == L or draft[t] != best:
            return len(out) - 1, out
    raise AssertionError


@pytest.mark.parametrize("set_id", range(6))
def test_greedy_verify_is_longest_matching_run(set_id):
    rng = np.random.default_rng(set_id)
    L, V, K = 5, 40, 4
    Z = np.round(rng.standard_normal((L + 1, V)) * 2) / 2      # ties included
    cand = np.stack([rng.permutation(V)[:K] for _ in range(L)])
    # make the drafts agree with the target for a random number of positions
    agree = int(rng.integers(0, L + 1))
    path = rng.integers(0, K, size=L)
    for t in range(agree):
        a = int(sorted(range(V), key=lambda i: (-Z[t, i], i))[0])
        row = [int(c) for c in cand[t]]
        if a in row:
            path[t] = row.index(a)
        else:
            cand[t, path[t]] = a
    q = np.eye(K)[path]
    n, out, _ = dflash.verify_stream(Z, cand, path, q, 0.0, 1, 0)
    n_ref, out_ref = _greedy_decode(Z, cand[np.arange(L), path])
    assert n == n_ref
    assert list(out[: n + 1]) == out_ref
    assert np.all(out[n + 1:] == -1)


def test_greedy_full_cycle_matches_decode():
    inp = synth.make(1, set_id=2)
    res = dflash.cycle_stream(inp, 0)
    Z = dflash.widen(inp["Z"][0], "f32")
    n_ref, out_ref = _greedy_decode(Z, res["draft_tok"])
    assert res["accept_len"] == n_ref and list(res["out_tok"][: n_ref + 1]) == out_ref


# ---------------------------------------------------------------- check (3)

def _tiny_stream(rng, L, V, K):
    Z = rng.standard_normal((L + 1, V)) * 1.5
    S = rng.standard_normal((L, K, K))
    S[0] = S[0][0][None, :]
    cand = np.stack([rng.permutation(V)[:K] for _ in range(L)])
    return Z, S, cand


def _emitted_by_position(Z, S, cand, T, n_cycles, seed, chunk):
    L = S.shape[0]
    emitted = [[] for _ in range(L + 1)]
    accepted_first = 0
    for c in range(n_cycles):
        path, draft, q, _ = dflash.trace_stream(S, cand, T, seed, c)
        n, out, _ = dflash.verify_stream(Z, cand, path, q, T, seed, c, chunk=chunk)
        for t in range(n + 1):
            emitted[t].append(int(out[t]))
        accepted_first += n >= 1
    return emitted, accepted_first


def _chi2_pvalue(tokens, p):
    counts = np.bincount(tokens, minlength=p.size).astype(float)
    exp = p * len(tokens)
    keep = exp >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    ex = np.append(exp[keep], exp[~keep].sum())
    if ex[-1] < 1e-9:
        obs, ex = obs[:-1], ex[:-1]
    return stats.chisquare(obs, ex).pvalue


@pytest.mark.parametrize("V,K,L,T,chunk", [
    (8, 2, 2, 1.0, 4096),
    (16, 4, 2, 0.7, 3),
    (12, 12, 1, 1.0, 1),
    (64, 16, 2, 1.3, 16),
])
def test_emitted_tokens_follow_target(V, K, L, T, chunk):
    rng = np.random.default_rng(V * 100 + K)
    Z, S, cand = _tiny_stream(rng, L, V, K)
    n_cycles = 6000
    emitted, _ = _emitted_by_position(Z, S, cand, T, n_cycles, 0x1234 + V, chunk)
    for t in range(L + 1):
        if len(emitted[t]) < 200:
            continue
        p = special.softmax(Z[t] / T)
        assert _chi2_pvalue(np.array(emitted[t]), p) > 1e-4, f"position {t + 1}"


@pytest.mark.parametrize("V,K,L,T,chunk", [
    (8, 2, 2, 1.0, 4096),
    (16, 4, 3, 0.7, 5),
    (64, 16, 2, 1.3, 16),
])
def test_one_hot_max_sum_proposal_keeps_target_law(V, K, L, T, chunk):
    # the max-sum path is deterministic, so its q is one-hot; the accept test
    # is then u < p(d) and the residual is p without d: the emitted token at
    # every position must still follow p, and position 1 is accepted with
    # probability sum(min(p, q)) = p(d_1)
    from oracle import viterbi
    rng = np.random.default_rng(V * 1000 + K + 7)
    Z, S, cand = _tiny_stream(rng, L, V, K)
    path, draft, _, _ = viterbi.viterbi_stream(S, cand)
    q = np.zeros((L, K))
    q[np.arange(L), path] = 1.0
    n_cycles = 6000
    emitted = [[] for _ in range(L + 1)]
    acc1 = 0
    for c in range(n_cycles):
        n, out, _ = dflash.verify_stream(Z, cand, path, q, T, 0x777 + V, c, chunk=chunk)
        for t in range(n + 1):
            emitted[t].append(int(out[t]))
        acc1 += n >= 1
    for t in range(L + 1):
        if len(emitted[t]) < 200:
            continue
        pt = special.softmax(Z[t] / T)
        assert _chi2_pvalue(np.array(emitted[t]), pt) > 1e-4, f"position {t + 1}"
    p1 = special.softmax(Z[0] / T)[int(draft[0])]
    sd = np.sqrt(p1 * (1 - p1) / n_cycles)
    assert abs(acc1 / n_cycles - p1) < 5 * sd + 1e-12


def test_first_position_acceptance_closed_form():
    rng = np.random.default_rng(77)
    V, K, L, T = 10, 3, 1, 1.0
    Z, S, cand = _tiny_stream(rng, L, V, K)
    n_cycles = 8000
    _, acc = _emitted_by_position(Z, S, cand, T, n_cycles, 4242, 4096)
    p = special.softmax(Z[0] / T)
    q_full = np.zeros(V)
    q_full[cand[0]] = special.softmax(S[0, 0] / T)
    want = np.minimum(p, q_full).sum()
    assert stats.binomtest(acc, n_cycles, want).pvalue > 1e-4


def test_q_equal_p_always_accepts_and_bonus_follows_last_row():
    rng = np.random.default_rng(5)
    V, L, T = 6, 2, 0.9
    Z = rng.standard_normal((L + 1, V))
    cand = np.stack([rng.permutation(V) for _ in range(L)])       # K = V
    S = np.stack([np.tile(Z[t, cand[t]], (V, 1)) for t in range(L)])
    bonus = []
    for c in range(3000):
        path, draft, q, _ = dflash.trace_stream(S, cand, T, 9, c)
        n, out, _ = dflash.verify_stream(Z, cand, path, q, T, 9, c)
        assert n == L
        bonus.append(int(out[L]))
    assert _chi2_pvalue(np.array(bonus), special.softmax(Z[L] / T)) > 1e-4


def test_residual_law_is_independent_of_chunk_size():
    # the two-level draw over (chunks, candidates) has the law of the
    # normalised residual for every chunk size; compare the residual draw
    # alone by forcing a rejection at position 1 (q(d) >> p(d))
    rng = np.random.default_rng(8)
    V, K, T = 20, 4, 1.0
    Z = rng.standard_normal((2, V))
    cand = rng.permutation(V)[:K][None, :]
    p = special.softmax(Z[0] / T)
    q = np.zeros((1, K))
    q[0] = [0.7, 0.1, 0.1, 0.1]
    resid = p.copy()
    resid[cand[0]] = np.maximum(0.0, p[cand[0]] - q[0])
    resid /= resid.sum()
    d_rank = np.array([int(np.argmax(q[0] - p[cand[0]]))])
    for chunk in (1, 6, 4096):
        toks = []
        for c in range(4000):
            n, out, _ = dflash.verify_stream(Z, cand, d_rank, q, T, 31, c, chunk=chunk)
            if n == 0:
                toks.append(int(out[0]))
        assert len(toks) > 1000
        assert _chi2_pvalue(np.array(toks), resid) > 1e-4, f"chunk {chunk}"


def test_degenerate_residual_falls_back_to_p():
    # q >= p on every candidate and no non-candidate mass (K = V): the
    # residual is identically zero, so the draw must come from p itself
    rng = np.random.default_rng(12)
    V, T = 5, 1.0
    Z = rng.standard_normal((2, V))
    cand = np.arange(V)[None, :]
    p = special.softmax(Z[0] / T)
    q = (2.0 * p)[None, :]
    toks = []
    for c in range(5000):
        n, out, _ = dflash.verify_stream(Z, cand, np.array([0]), q, T, 2, c)
        if n == 0:
            toks.append(int(out[0]))
    assert len(toks) > 1000
    assert _chi2_pvalue(np.array(toks), p) > 1e-4


@pytest.mark.parametrize("T", [-1.0, -1e-30, float("nan")])
def test_non_positive_or_nan_temperature_is_greedy(T):
    # the library's rule (T > 0 samples, every other value is greedy) taken
    # by the oracle: the cycle then equals the T = 0 cycle, and its verify is
    # the longest run matching the target argmax
    a = synth.make(3, set_id=21, B=2, V=4096, hidden=64, T=0.0)
    b = synth.make(3, set_id=21, B=2, V=4096, hidden=64, T=T)
    for s in range(2):
        ra, rb = dflash.cycle_stream(a, s), dflash.cycle_stream(b, s)
        for k in ("path_rank", "draft_tok", "q", "out_tok"):
            np.testing.assert_array_equal(ra[k], rb[k], err_msg=k)
        assert ra["accept_len"] == rb["accept_len"]
        Z = dflash.widen(b["Z"][s], "bf16")
        n_ref, out_ref = _greedy_decode(Z, rb["draft_tok"])
        assert rb["accept_len"] == n_ref and list(rb["out_tok"][: n_ref + 1]) == out_ref


# ---------------------------------------------------------------- vocabulary split

def test_chunk_bounds_partition_the_vocabulary():
    # the items always cover every token once, in index order, and never
    # straddle a shard boundary
    for V, chunk, begins in ((151936, 4096, None), (151936, 4096, [0, 18992, 37984, 56976, 75968, 94960,
                                                                    113952, 132944]),
                             (100, 7, [0, 13, 14, 60]), (64, 8, [0])):
        b = dflash.chunk_bounds(V, chunk, begins)
        assert b[0][0] == 0 and b[-1][1] == V
        assert all(b[i][1] == b[i + 1][0] for i in range(len(b) - 1))
        assert all(0 < hi - lo <= chunk for lo, hi in b)
        for s in (begins or [0]):
            assert any(lo == s for lo, _ in b)


def test_aligned_or_single_shard_split_changes_nothing():
    # shard boundaries on the chunk grid (262144 / 8) or a single shard give
    # the unsplit chunks, so every output is identical
    inp = synth.make(5, set_id=31, B=3, V=32768, hidden=64)
    for begins in ([0], [0, 4096, 8192, 12288, 16384, 20480, 24576, 28672]):
        for s in range(inp["B"]):
            a, b = dflash.cycle_stream(inp, s), dflash.cycle_stream(inp, s, shard_begin=begins)
            assert a["accept_len"] == b["accept_len"]
            np.testing.assert_array_equal(a["out_tok"], b["out_tok"])


def test_ragged_split_moves_only_the_in_chunk_draw():
    # with shard boundaries off the grid the chunks differ, so the token a
    # given uniform lands on may differ, but only through the residual draw:
    # the candidates, path, q and accept count never change
    inp = synth.make(3, set_id=32, B=4, V=20008, hidden=64)
    begins = [0, 2501, 5002, 7503, 10004, 12505, 15006, 17507]
    for s in range(inp["B"]):
        a, b = dflash.cycle_stream(inp, s), dflash.cycle_stream(inp, s, shard_begin=begins)
        for k in ("cand_idx", "path_rank", "draft_tok", "q"):
            np.testing.assert_array_equal(a[k], b[k])
        assert a["accept_len"] == b["accept_len"]
        np.testing.assert_array_equal(a["out_tok"][: a["accept_len"]], b["out_tok"][: b["accept_len"]])


@pytest.mark.parametrize("begins", [[0, 7], [0, 3, 11, 17], [0, 1, 2, 19]])
def test_residual_law_is_unchanged_by_a_vocabulary_split(begins):
    # the residual draw over a chunk grid that restarts at each shard
    # boundary still follows the normalised residual (forced rejection at
    # position 1, as in the chunk-size test)
    rng = np.random.default_rng(18)
    V, K, T = 20, 4, 1.0
    Z = rng.standard_normal((2, V))
    cand = rng.permutation(V)[:K][None, :]
    p = special.softmax(Z[0] / T)
    q = np.zeros((1, K))
    q[0] = [0.7, 0.1, 0.1, 0.1]
    resid = p.copy()
    resid[cand[0]] = np.maximum(0.0, p[cand[0]] - q[0])
    resid /= resid.sum()
    d_rank = np.array([int(np.argmax(q[0] - p[cand[0]]))])
    toks = []
    for c in range(4000):
        n, out, _ = dflash.verify_stream(Z, cand, d_rank, q, T, 37, c, chunk=4, shard_begin=begins)
        if n == 0:
            toks.append(int(out[0]))
    assert len(toks) > 1000
    assert _chi2_pvalue(np.array(toks), resid) > 1e-4


def test_bonus_law_is_unchanged_by_a_vocabulary_split():
    # the bonus row has no candidates: the two-level draw over the split
    # chunk grid must follow p of the last row
    rng = np.random.default_rng(6)
    V, L, T = 24, 1, 0.8
    Z = rng.standard_normal((L + 1, V))
    cand = np.stack([rng.permutation(V) for _ in range(L)])
    S = np.stack([np.tile(Z[t, cand[t]], (V, 1)) for t in range(L)])
    bonus = []
    for c in range(3000):
        path, draft, q, _ = dflash.trace_stream(S, cand, T, 3, c)
        n, out, _ = dflash.verify_stream(Z, cand, path, q, T, 3, c, chunk=5, shard_begin=[0, 9, 10, 17])
        assert n == L
        bonus.append(int(out[L]))
    assert _chi2_pvalue(np.array(bonus), special.softmax(Z[L] / T)) > 1e-4
