"""Pins of the lattice wiring in ``oracle.dflash.cycle_stream``.

P3 "DFlash 2: Keep Drafting Parallel", section "What Comes Next", paragraph
"A Lightweight Path Selector": every edge scores a predecessor a (the
previous position's candidate, the verified token for the first edge)
against a current candidate b, with the drafter's logit of b and an
embedding match under the gate of the current position's context h_t.

The unit pins of ``gate`` and ``pair_scores`` do not fix which rows feed
which edge.  Here a tiny lattice is built by hand so that every score has a
closed form: each embedding row is a scaled one-hot vector, E[v] = c_v e_(v mod
r), so the bilinear term of (a, b) is c_a c_b g_t[a mod r] when a and b share
a residue and 0 otherwise; the gate weights read only the first context
entry, g_t[k] = sigmoid(w_k h_t[0]), with h_t[0] different at every position;
the drafter rows put four hand-chosen candidates on top in a known order.
The residues are chosen so that each plausible wiring mistake (gating edge t
with h_(t-1), taking predecessors from C_t, using x0 past the first edge,
adding the drafter logit by row) changes some score, and each such mistake,
planted into a copy of the composition, is shown to fail the pin.
"""

import math

import numpy as np

from oracle import dflash as O

V, K, R, H, L = 64, 4, 16, 16, 3
CANDS = [[5, 22, 39, 56], [21, 6, 55, 40], [7, 23, 38, 53]]
X0 = 37
HT0 = [0.7, -1.4, 2.1]          # h_t[0] per position
W0 = [0.1 * (k + 1) for k in range(R)]


def c_of(v):
    return 0.5 + v / 64.0


def _inputs(T=0.0):
    U = np.empty((1, L, V), dtype=np.float32)
    for t in range(L):
        U[0, t] = -1.0 - 0.01 * np.arange(V, dtype=np.float32)
        for j, v in enumerate(CANDS[t]):
            U[0, t, v] = 10.0 - j - 0.25 * t
    E = np.zeros((V, R), dtype=np.float32)
    for v in range(V):
        E[v, v % R] = c_of(v)
    W = np.zeros((R, H), dtype=np.float32)
    W[:, 0] = W0
    rng = np.random.default_rng(5)
    h = rng.standard_normal((1, L, H)).astype(np.float32)
    h[0, :, 0] = HT0
    Z = np.concatenate([U, U[:, :1] * 0.5], axis=1)
    return dict(B=1, L=L, V=V, K=K, r=R, hidden=H, logit_kind="f32", param_kind="f32",
                U=U, Z=Z, x0=np.array([X0], dtype=np.int32), E=E, W=W, h=h,
                T=np.array([T], dtype=np.float32), seed=np.array([7], dtype=np.uint64), cycle=3)


def _sig(x):
    return 1.0 / (1.0 + math.exp(-x))


def closed_form_scores():
    """S[t][i][j] from the hand-built structure: drafter logit of candidate
    j, plus c_a c_b g_t[residue] when predecessor a and candidate b share a
    residue (a = x0 at the first edge, a = C_(t-1)[i] after it)."""
    inp = _inputs()
    S = np.zeros((L, K, K))
    for t in range(L):
        g = [_sig(float(np.float32(W0[k])) * float(np.float32(HT0[t]))) for k in range(R)]
        for i in range(K):
            a = X0 if t == 0 else CANDS[t - 1][i]
            for j in range(K):
                b = CANDS[t][j]
                s = float(inp["U"][0, t, b])
                if a % R == b % R:
                    s += c_of(a) * c_of(b) * g[a % R]
                S[t, i, j] = s
    return S


def _mutant_scores(inp, mistake):
    """The composition of cycle_stream with one wiring mistake planted,
    built from the oracle's own gate and pair_scores."""
    U = O.widen(inp["U"][0], "f32")
    ci = np.stack([O.topk_row(U[t], K)[0] for t in range(L)])
    cv = np.stack([O.topk_row(U[t], K)[1] for t in range(L)])
    E, W, h = (O.widen(inp[k], "f32") for k in ("E", "W", "h"))
    S = np.zeros((L, K, K))
    for t in range(L):
        th = max(t - 1, 0) if mistake == "gate_prev_h" else t
        g = O.gate(h[0, th], W)
        if t == 0 or mistake == "x0_everywhere":
            pred = np.repeat(E[int(inp["x0"][0])][None, :], K, axis=0)
        elif mistake == "pred_from_current":
            pred = E[ci[t]]
        else:
            pred = E[ci[t - 1]]
        S[t] = O.pair_scores(pred, E[ci[t]], cv[t], g)
        if mistake == "logit_by_row":
            S[t] = S[t] - cv[t][None, :] + cv[t][:, None]
    return S


MISTAKES = ["gate_prev_h", "pred_from_current", "x0_everywhere", "logit_by_row"]


def test_candidates_are_the_planted_ones():
    r = O.cycle_stream(_inputs(), 0)
    np.testing.assert_array_equal(r["cand_idx"], np.array(CANDS))


def test_scores_follow_the_wiring():
    r = O.cycle_stream(_inputs(), 0)
    np.testing.assert_allclose(r["S"], closed_form_scores(), rtol=0, atol=1e-12)


def test_greedy_path_follows_the_closed_form():
    S = closed_form_scores()
    prev, path = 0, []
    for t in range(L):
        row = S[t, prev]
        prev = int(np.flatnonzero(row == row.max())[0])
        path.append(prev)
    r = O.cycle_stream(_inputs(), 0)
    np.testing.assert_array_equal(r["path_rank"], path)
    np.testing.assert_array_equal(r["draft_tok"], [CANDS[t][path[t]] for t in range(L)])


def test_lattice_makes_the_pin_bite():
    # the residues put matching pairs on every edge and the predecessor
    # sets differ from edge to edge, so the bilinear term is active where
    # each mistake would move it
    S = closed_form_scores()
    U = _inputs()["U"][0]
    for t in range(L):
        assert np.any(S[t] != U[t][CANDS[t]][None, :]), t


def test_every_planted_wiring_mistake_fails_the_pin():
    S = closed_form_scores()
    inp = _inputs()
    np.testing.assert_allclose(_mutant_scores(inp, None), S, rtol=0, atol=1e-12)
    for m in MISTAKES:
        diff = np.abs(_mutant_scores(inp, m) - S).max()
        assert diff > 1e-3, (m, diff)
