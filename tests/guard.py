"""Near-tie margin guard for parity inputs.

The HIP path decides argmaxes, accept tests and inverse-CDF draws on fp32
(streaming sums, scores) and fp64 (finalize) values; the oracle decides them
in fp64.  Two correct implementations can disagree only when a decision is
closer to its boundary than their rounding differences.  The guard runs the
oracle on an input set, reads the margin of every decision it took, and
re-draws the stream's Philox seed (sampling decisions) or context vector h
(greedy trace ties) until every margin clears its threshold.

Thresholds (relative to the stated scale):
  trace_gap  1e-5 * max(1, |best score|)   fp32 score error is ~1e-7 relative
  trace_cdf  1e-5 * total weight * sens_t   fp32 scores enter exp()
  accept     1e-5 * max(u q, p) * sens_t    fp32 row sums (~1e-6 relative), q
  item_cdf   1e-5 (probability units)       fp32 chunk sums
  chunk_cdf  1e-5 * chunk mass              fp32 weights (v_exp_f32) inside a
                                            chunk, fp64 sums (~2e-7 relative)

sens_t = max(1, 0.1 * max |S row| / T) at a sampled position t: the GPU's
scores are fp32, so each carries an absolute error up to about 2^-23 |S|,
which the trace's softmax turns into a relative error of about 2^-22 |S| / T
in every weight of the row and in q_t; with large scores at a low
temperature (|S| / T in the hundreds) that exceeds the plain 1e-5.
"""

import numpy as np

from oracle import dflash

THRESH = {"trace_gap": 1e-5, "trace_cdf": 1e-5, "accept": 1e-5, "item_cdf": 1e-5, "chunk_cdf": 1e-5}


def score_sensitivity(r):
    """sens_t of every drafted position of one oracle result (1 when greedy)."""
    T, S, path = r["T"], r["S"], r["path_rank"]
    sens, prev = [], 0
    for t in range(S.shape[0]):
        sens.append(max(1.0, 0.1 * float(np.abs(S[t, prev]).max()) / T) if T > 0 else 1.0)
        prev = int(path[t])
    return sens


def violations(margins, sens=None):
    """Margins closer than their threshold.  The trace_cdf and accept
    margins come in position order (one per drafted position reached), so
    the i-th of each kind is scaled by sens[i]."""
    bad, seen = [], {"trace_cdf": 0, "accept": 0}
    for (k, v, s) in margins:
        f = 1.0
        if sens is not None and k in seen:
            f = sens[min(seen[k], len(sens) - 1)]
            seen[k] += 1
        if v < THRESH[k] * s * f:
            bad.append((k, v, s))
    return bad


def _redraw_h(inp, b, attempt):
    rng = np.random.default_rng([int(inp["config_id"]), int(inp["set_id"]), int(b), 7000 + attempt])
    x = rng.standard_normal(inp["h"][b].shape, dtype=np.float32)
    if inp["param_kind"] == "bf16":
        import synth
        inp["h"][b] = synth.bf16_bits(x)
    else:
        inp["h"][b] = x


def guarded(inp, streams=None, max_tries=40, guard_trace=True, shard_begin=None):
    """Oracle results for ``streams`` with every decision clear of the guard
    (``shard_begin``: the vocabulary split of the residual draw's chunks).

    Mutates ``inp`` (seed[b] and possibly h[b]) for re-drawn streams and
    returns (results dict by stream, number of re-draws).
    """
    if streams is None:
        streams = range(int(inp["B"]))
    res, redraws = {}, 0
    for b in streams:
        b = int(b)
        for attempt in range(max_tries):
            r = dflash.cycle_stream(inp, b, shard_begin=shard_begin)
            bad = violations(r["margins"], score_sensitivity(r))
            if not guard_trace:
                bad = [x for x in bad if x[0] != "trace_gap"]
            if not bad:
                break
            redraws += 1
            if any(k == "trace_gap" for k, _, _ in bad):
                _redraw_h(inp, b, attempt)
            else:
                inp["seed"][b] = np.uint64((int(inp["seed"][b]) + (1 << 48) * (attempt + 1)) & 0xFFFFFFFFFFFFFFFF)
        else:
            raise RuntimeError(f"stream {b}: no guard-clean input after {max_tries} draws")
        res[b] = r
    return res, redraws
