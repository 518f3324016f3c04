"""Plain float64 oracle of one DFlash 2 draft -> select -> verify cycle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Shares no code with
the HIP library and imports nothing from it.

Sources (four web pages on DFlash 2; cited by page title and section):
  P1  "DFlash 2: Block diffusion, wearing a drafter's coat"
      (skandtandon.pages.dev), section "The architecture": sub-sections
      "Sixteen candidates per position", "A path selector", "Lossless, with
      conditions I did not used to state".
  P2  "A 2B Drafter Made a 27B Model 3.4x Faster. Same Exact Output."
      (aibacon.net), sections "What a block-diffusion drafter is, and why it
      kept breaking", "The two fixes", "Caveats before you rebuild your
      serving stack".
  P3  "DFlash 2: Keep Drafting Parallel" news text (gab.ae), section "What
      Comes Next", figure text and paragraph "A Lightweight Path Selector".

Notation.  One stream has a block of L drafted positions t = 1..L.  U_t is
the drafter's logit row at position t (length V), h_t its context vector, x0
the last verified token.  Z_t (t = 1..L+1) are the target's logit rows.
C_t is the ordered list of K candidates at position t.  E is the [V, r]
candidate-embedding table and W the [r, hidden] gate matrix (one row per
embedding dimension, the layout of a linear layer's weight).

Readings of points the pages leave open:
  * score:   s_t(a, b) = U_t(b) + sum_k E[a,k] * g_t[k] * E[b,k],
             g_t = sigmoid(W @ h_t)  (the formula itself was lost from P3);
  * edge 1 uses a = x0 for every row of its score matrix;
  * trace:   greedy left-to-right walk (T = 0) or a draw from
             softmax(s_t(a_{t-1}, .) / T) over C_t (T > 0); q_t is that
             softmax (one-hot at T = 0);
  * verify:  accept position t while u * q_t(d_t) < p_t(d_t); at the first
             rejection draw from the normalised max(0, p - q) (candidates) /
             p (all other tokens); if all L are accepted, draw a bonus token
             from p_{L+1}; T = 0 replaces every draw by the argmax;
  * one temperature per stream for both the selector and the target; a
    stream samples when T > 0 and is greedy for every other value (0,
    negative, NaN);
  * the residual draw is a two-level inverse CDF: first over items
             [chunk 0 .. chunk n_c-1, candidate 0 .. K-1] (chunks of CHUNK
             tokens in index order, carrying the non-candidate mass), then,
             if a chunk was drawn, over the non-candidate tokens inside it.
"""

import math

import numpy as np

from . import philox

CHUNK = 4096            # tokens per first-level item of the residual draw


# --------------------------------------------------------------------------
# storage -> float64
# --------------------------------------------------------------------------

def widen(x, kind):
    """Exact float64 value of stored elements.

    ``kind`` is "bf16" (``x`` holds the 16-bit patterns as uint16) or "f32".
    A bf16 pattern is the upper half of a float32, so shifting it left by 16
    bits gives the float32 of identical value.
    """
    if kind == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if kind == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown storage kind {kind!r}")


# --------------------------------------------------------------------------
# S1: top-K candidates (P1 "Sixteen candidates per position";
#     P2 "What a block-diffusion drafter is ...", selection headroom)
# --------------------------------------------------------------------------

def topk_row(u_row, K):
    """The K tokens of one drafter row with the largest logits.

    Ordered by value (descending), equal values by token index (ascending);
    -0.0 and +0.0 compare equal.  A full lexicographic sort of all V tokens.
    Returns (indices int64[K], values float64[K]).
    """
    v = np.asarray(u_row, dtype=np.float64)
    order = np.lexsort((np.arange(v.size), -v))
    sel = order[:K]
    return sel.astype(np.int64), v[sel]


# --------------------------------------------------------------------------
# S2: context gate (P3 "A Lightweight Path Selector": embeddings matched
#     under a context gate H(h_t))
# --------------------------------------------------------------------------

def gate(h_t, W):
    """g_t = sigmoid(W @ h_t): one gate weight per embedding dimension.

    ``W`` is [r, hidden]; row k holds the weights of gate dimension k.
    """
    a = np.asarray(W, dtype=np.float64) @ np.asarray(h_t, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-a))


# --------------------------------------------------------------------------
# S3: adjacent pair scores (P3 "A Lightweight Path Selector"; P1 "A path
#     selector": neighbouring positions' candidates matched through a gated
#     bilinear form of small rank)
# --------------------------------------------------------------------------

def pair_scores(pred_emb, cand_emb, cand_val, g):
    """Score matrix of one edge.

    S[i, j] = U_t(b_j) + sum_k pred_emb[i, k] * g[k] * cand_emb[j, k]
    where row i is the i-th predecessor candidate and column j the j-th
    candidate at this position.  Parity unpinned against the pages: the
    pages keep the two terms (the drafter's own logit and a gated bilinear
    match of two r-dimensional embeddings) but lost the formula itself.
    """
    pred_emb = np.asarray(pred_emb, dtype=np.float64)
    cand_emb = np.asarray(cand_emb, dtype=np.float64)
    return np.asarray(cand_val, dtype=np.float64)[None, :] + (pred_emb * g[None, :]) @ cand_emb.T


# --------------------------------------------------------------------------
# helpers for inverse-CDF draws
# --------------------------------------------------------------------------

def _first_above(cum, target):
    """Smallest index j with cum[j] > target (cum non-decreasing, target < cum[-1])."""
    hits = np.flatnonzero(cum > target)
    return int(hits[0])


def _cdf_margin(cum, j, target):
    """Distance from ``target`` to the boundaries that decide index ``j``.

    The lower boundary cum[j-1] matters for j > 0, the upper one cum[j] for
    j < last (the last cumulative value is the total itself, against which
    target = u * total < total can never flip).
    """
    d = math.inf
    if j > 0:
        d = min(d, target - cum[j - 1])
    if j < len(cum) - 1:
        d = min(d, cum[j] - target)
    return d


# --------------------------------------------------------------------------
# S4: trace (P3 "A Lightweight Path Selector": once the scores exist, only
#     a walk from the verified token is left in sequence; at T = 0 it takes
#     the highest-scoring next candidate, at T > 0 it draws the next one
#     from the scores)
# --------------------------------------------------------------------------

def trace_stream(S, cand_idx, T, seed, cycle):
    """Walk one path through the candidate lattice of one stream.

    ``S`` is [L, K, K] (edge t: rows = predecessor rank, cols = candidate
    rank), ``cand_idx`` is [L, K].  Row 0 is used at edge 1 (all rows of
    edge 1 are equal, its predecessor being x0).

    T <= 0 or NaN (greedy): j_t = smallest rank attaining the maximum of
           S[t, j_{t-1}, :]; q_t is one-hot at j_t.
    T > 0: w = exp((row - max row) / T), q_t = w / sum(w); with u the fp32
           uniform from word 0 of the (seed; cycle, t, 0) Philox block,
           j_t = smallest rank whose cumulative weight exceeds u * total.

    Returns (path_rank int64[L], draft_tok int64[L], q float64[L, K],
    margins list of (kind, value, scale)).
    """
    S = np.asarray(S, dtype=np.float64)
    L, K, _ = S.shape
    path = np.zeros(L, dtype=np.int64)
    q = np.zeros((L, K), dtype=np.float64)
    margins = []
    prev = 0
    for t in range(L):
        row = S[t, prev, :]
        if T > 0:
            m = row.max()
            w = np.exp((row - m) / T)
            cum = np.cumsum(w)
            total = cum[-1]
            u = philox.u01_f32(philox.stream_block(seed, cycle, t + 1, 0)[0])
            target = u * total
            j = _first_above(cum, target)
            q[t] = w / total
            margins.append(("trace_cdf", _cdf_margin(cum, j, target), total))
        else:
            best = row.max()
            j = int(np.flatnonzero(row == best)[0])
            q[t, j] = 1.0
            rest = np.delete(row, j)
            gap = best - rest.max() if rest.size else math.inf
            margins.append(("trace_gap", gap, max(1.0, abs(best))))
        path[t] = j
        prev = j
    draft = np.asarray(cand_idx)[np.arange(L), path].astype(np.int64)
    return path, draft, q, margins


# --------------------------------------------------------------------------
# S5 + S6: verify against the target (P1 "Lossless, with conditions ...":
#     a draft survives with chance min(1, p/q), and a rejected one is
#     replaced by a draw from the residual; P2 "Caveats ...": greedy output
#     equals the target's)
# --------------------------------------------------------------------------

def argmax_first(row):
    """Smallest index attaining the maximum of a row."""
    row = np.asarray(row, dtype=np.float64)
    return int(np.flatnonzero(row == row.max())[0])


def softmax_T(z, T):
    """p = exp((z - max z) / T) / sum, in float64."""
    z = np.asarray(z, dtype=np.float64)
    w = np.exp((z - z.max()) / T)
    return w / w.sum()


def chunk_bounds(V, chunk=CHUNK, shard_begin=None):
    """The first-level items of the residual draw: (lo, hi) token ranges.

    Without a vocabulary split the tokens are cut into runs of ``chunk`` in
    index order (the last one shorter).  With one (P1 "DFlash 2: Block
    diffusion, wearing a drafter's coat", "The architecture", "Parallel
    block drafting", and the serving runtimes of P2 "A 2B Drafter Made a
    27B Model 3.4x Faster. Same Exact Output.", "Running it", where the
    target's vocabulary may be split across devices) the cut restarts at
    every shard boundary, so that no chunk straddles two shards: shard s
    covers [shard_begin[s], shard_begin[s+1]) (the last up to V) and is cut
    into runs of ``chunk`` from its own first token.  This build's reading:
    the draw only needs the items to partition the tokens in index order,
    so any such cut leaves the residual law unchanged.
    """
    starts = [0] if shard_begin is None else [int(s) for s in shard_begin]
    ends = starts[1:] + [V]
    out = []
    for lo_s, hi_s in zip(starts, ends):
        for lo in range(lo_s, hi_s, chunk):
            out.append((lo, min(lo + chunk, hi_s)))
    return out


def verify_stream(Zrows, cand_idx, path_rank, q, T, seed, cycle, chunk=CHUNK, shard_begin=None):
    """Rejection-sampling verify of one stream's drafted path.

    ``Zrows`` [L+1, V] target logits (float64), ``cand_idx`` [L, K],
    ``path_rank`` [L], ``q`` [L, K] the drafting distribution over each
    position's candidates.

    T <= 0 or NaN (greedy): a_t = argmax_first(Z_t); n = length of the
           longest prefix with d_t == a_t; the emitted tokens are
           d_1..d_n, a_{n+1}.
    T > 0: p_t = softmax(Z_t / T).  Position t is accepted while
           u_t * q_t(d_t) < p_t(d_t), u_t the fp32 uniform from word 1 of
           the (seed; cycle, t, 0) block.  n = number accepted.  Row n+1 is
           the sampling row: if n < L its residual is max(0, p - q) on the
           candidates of position n+1 and p elsewhere; if n = L it is
           p_{L+1} with no candidates.  If the residual's total is not
           positive it is replaced by p (candidates keep mass p).  The draw
           uses the fp64 uniforms u1 (words 0,1) and u2 (words 2,3) of the
           (seed; cycle, n+1, 1) block: u1 picks an item among
           [chunk 0..n_c-1 (non-candidate mass), candidate 0..K-1], u2 picks
           a non-candidate token inside a picked chunk.  The chunks are those
           of :func:`chunk_bounds` (``shard_begin``: a vocabulary split).

    Returns (accept_len, out_tok int64[L+1] padded with -1, margins).
    """
    Z = np.asarray(Zrows, dtype=np.float64)
    Lp1, V = Z.shape
    L = Lp1 - 1
    cand_idx = np.asarray(cand_idx, dtype=np.int64)
    path_rank = np.asarray(path_rank, dtype=np.int64)
    q = np.asarray(q, dtype=np.float64)
    draft = cand_idx[np.arange(L), path_rank]
    out = np.full(L + 1, -1, dtype=np.int64)
    margins = []

    if not T > 0:
        # greedy: T = 0 by the pages' convention, and by this build's reading
        # every temperature that is not positive (negative or NaN) as well
        a = [argmax_first(Z[t]) for t in range(L + 1)]
        n = 0
        while n < L and draft[n] == a[n]:
            n += 1
        out[:n] = draft[:n]
        out[n] = a[n]
        return n, out, margins

    P = np.stack([softmax_T(Z[t], T) for t in range(L + 1)])
    n = L
    for t in range(L):
        u = philox.u01_f32(philox.stream_block(seed, cycle, t + 1, 0)[1])
        lhs = u * q[t, path_rank[t]]
        rhs = P[t, draft[t]]
        margins.append(("accept", abs(lhs - rhs), max(lhs, rhs)))
        if not lhs < rhs:
            n = t
            break

    row = n                                  # 0-based index of the sampling row
    p = P[row]
    if n < L:
        cand = cand_idx[row]
        cand_mass = np.maximum(0.0, p[cand] - q[row])
    else:
        cand = np.zeros(0, dtype=np.int64)
        cand_mass = np.zeros(0)
    r = p.copy()
    r[cand] = 0.0                            # non-candidate mass only
    bounds = chunk_bounds(V, chunk, shard_begin)
    n_c = len(bounds)
    chunk_mass = np.array([r[lo:hi].sum() for lo, hi in bounds])
    items = np.concatenate([chunk_mass, cand_mass])
    if not items.sum() > 0:
        items = np.concatenate([chunk_mass, p[cand]])

    w = philox.stream_block(seed, cycle, row + 1, 1)
    u1 = philox.u01_f64(w[0], w[1])
    u2 = philox.u01_f64(w[2], w[3])
    cum = np.cumsum(items)
    target = u1 * cum[-1]
    m = _first_above(cum, target)
    margins.append(("item_cdf", _cdf_margin(cum, m, target), 1.0))
    if m >= n_c:
        tok = int(cand[m - n_c])
    else:
        lo, hi = bounds[m]
        seg = r[lo:hi]
        cs = np.cumsum(seg)
        tgt = u2 * cs[-1]
        i = _first_above(cs, tgt)
        margins.append(("chunk_cdf", _cdf_margin(cs, i, tgt), cs[-1]))
        tok = lo + i
    out[:n] = draft[:n]
    out[n] = tok
    return n, out, margins


# --------------------------------------------------------------------------
# one whole cycle of one stream, and of a batch
# --------------------------------------------------------------------------

def cycle_stream(inp, b, chunk=CHUNK, shard_begin=None):
    """All steps S1..S6 for stream ``b`` of an input set.

    ``inp`` is a mapping with keys B, L, V, K, r, hidden, logit_kind,
    param_kind, U [B,L,V], Z [B,L+1,V], x0 [B], E [V,r], W [r,hidden],
    h [B,L,hidden], T [B], seed [B], cycle (int).  Arrays hold storage
    values (uint16 bf16 patterns or float32); everything is widened here.
    ``shard_begin``: the first tokens of a vocabulary split, which moves the
    residual draw's chunk boundaries (:func:`chunk_bounds`); the candidates,
    scores and path do not depend on it.
    """
    L, K = int(inp["L"]), int(inp["K"])
    lk, pk = inp["logit_kind"], inp["param_kind"]
    T = float(np.float32(inp["T"][b]))
    seed = int(inp["seed"][b])
    cyc = int(inp["cycle"])

    U = widen(inp["U"][b], lk)                       # [L, V]
    cand_idx = np.zeros((L, K), dtype=np.int64)
    cand_val = np.zeros((L, K))
    for t in range(L):
        cand_idx[t], cand_val[t] = topk_row(U[t], K)

    W = widen(inp["W"], pk)
    S = np.zeros((L, K, K))
    for t in range(L):
        g = gate(widen(inp["h"][b, t], pk), W)
        if t == 0:
            pred = np.repeat(widen(inp["E"][int(inp["x0"][b])][None, :], pk), K, axis=0)
        else:
            pred = widen(inp["E"][cand_idx[t - 1]], pk)
        cand_emb = widen(inp["E"][cand_idx[t]], pk)
        S[t] = pair_scores(pred, cand_emb, cand_val[t], g)

    path, draft, q, m_trace = trace_stream(S, cand_idx, T, seed, cyc)
    Zr = widen(inp["Z"][b], lk)                      # [L+1, V]
    n, out, m_verify = verify_stream(Zr, cand_idx, path, q, T, seed, cyc, chunk=chunk, shard_begin=shard_begin)
    return {
        "cand_idx": cand_idx, "cand_val": cand_val, "S": S,
        "path_rank": path, "draft_tok": draft, "q": q,
        "accept_len": n, "out_tok": out, "T": T,
        "margins": m_trace + m_verify,
    }


def cycle(inp, streams=None, chunk=CHUNK, shard_begin=None):
    """:func:`cycle_stream` for every stream in ``streams`` (default: all)."""
    if streams is None:
        streams = range(int(inp["B"]))
    return {int(b): cycle_stream(inp, int(b), chunk=chunk, shard_begin=shard_begin) for b in streams}
