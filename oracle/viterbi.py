"""Plain float64 oracle of the global max-sum (Viterbi) path through the
candidate lattice.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Shares no code with
the HIP library and imports nothing from it.

Source: P3 "DFlash 2: Keep Drafting Parallel", section "What Comes Next",
paragraph "A Lightweight Path Selector": the selector scores every adjacent
candidate pair and its greedy trace follows the best successor from the
verified token; the same section leaves better searches open.  This variant
keeps the pair scores and replaces the left-to-right greedy walk by the path
whose summed edge scores are largest over all K^L paths.

Reading of what the pages leave open:
  * the path's value is the plain sum of its L edge scores
    S[0, 0, j_1] + S[1, j_1, j_2] + ... + S[L-1, j_{L-1}, j_L] (edge 1 starts
    at the verified token, whose K rows are equal, so row 0 stands for it);
  * among paths of equal value the one taken is the smallest in reverse
    lexicographic order, comparing j_L first, then j_{L-1}, and so on;
  * the path is deterministic, so its proposal distribution q_t is one-hot at
    the chosen rank; rejection sampling against the target stays exact for a
    one-hot proposal at any temperature.
"""

import numpy as np


def viterbi_stream(S, cand_idx):
    """Max-sum path of one stream.

    ``S`` is [L, K, K] (edge t: rows = predecessor rank, cols = candidate
    rank), ``cand_idx`` is [L, K].  Dynamic programming in float64:
    best_1(j) = S[0, 0, j]; best_t(j) = max_i best_{t-1}(i) + S[t-1, i, j],
    with back_t(j) the smallest i attaining it; j_L = smallest j attaining
    max best_L(j); then j_{t-1} = back_t(j_t).  Taking the smallest index at
    every tie gives the reverse-lexicographically smallest optimal path.

    Returns (path_rank int64[L], draft_tok int64[L], value float64, margins
    list of (kind, value, scale)), the margins being the gap between the
    chosen and the runner-up option of every decision the backtrack reads.

    Pinned by ``tests/test_oracle_viterbi.py``: brute-force enumeration of
    all K^L paths (value and tie rule, integer scores with many ties),
    independent top-1 picks when the scores do not depend on the
    predecessor, one position, a hand-built lattice where greedy and
    max-sum differ, invariance to a constant added to one edge.
    """
    S = np.asarray(S, dtype=np.float64)
    L, K, _ = S.shape
    best = S[0, 0, :].copy()
    back = np.zeros((L, K), dtype=np.int64)
    gaps = np.full((L, K), np.inf)
    for t in range(1, L):
        cand = best[:, None] + S[t]                     # [i, j]
        nb = np.empty(K)
        for j in range(K):
            col = cand[:, j]
            m = col.max()
            i = int(np.flatnonzero(col == m)[0])
            back[t, j] = i
            nb[j] = m
            rest = np.delete(col, i)
            gaps[t, j] = m - rest.max() if rest.size else np.inf
        best = nb
    top = best.max()
    jl = int(np.flatnonzero(best == top)[0])
    rest = np.delete(best, jl)
    margins = [("trace_gap", top - rest.max() if rest.size else np.inf, max(1.0, abs(top)))]
    path = np.zeros(L, dtype=np.int64)
    path[L - 1] = jl
    for t in range(L - 1, 0, -1):
        j = path[t]
        margins.append(("trace_gap", gaps[t, j], max(1.0, abs(best.max()))))
        path[t - 1] = back[t, j]
    draft = np.asarray(cand_idx)[np.arange(L), path].astype(np.int64)
    return path, draft, float(top), margins


def path_value(S, path):
    """Summed edge scores of one path (row 0 at edge 1)."""
    S = np.asarray(S, dtype=np.float64)
    prev, v = 0, 0.0
    for t, j in enumerate(path):
        v += S[t, prev, j]
        prev = j
    return v
