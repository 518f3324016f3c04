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
  trace_cdf  1e-5 * total weight            fp32 scores enter exp()
  accept     1e-5 * max(u q, p)             fp32 row sums (~1e-6 relative)
  item_cdf   1e-5 (probability units)       fp32 chunk sums
  chunk_cdf  1e-9 * chunk mass              both sides fp64
"""

import numpy as np

from oracle import dflash

THRESH = {"trace_gap": 1e-5, "trace_cdf": 1e-5, "accept": 1e-5, "item_cdf": 1e-5, "chunk_cdf": 1e-9}


def violations(margins):
    return [(k, v, s) for (k, v, s) in margins if v < THRESH[k] * s]


def _redraw_h(inp, b, attempt):
    rng = np.random.default_rng([int(inp["config_id"]), int(inp["set_id"]), int(b), 7000 + attempt])
    x = rng.standard_normal(inp["h"][b].shape, dtype=np.float32)
    if inp["param_kind"] == "bf16":
        import synth
        inp["h"][b] = synth.bf16_bits(x)
    else:
        inp["h"][b] = x


def guarded(inp, streams=None, max_tries=40, guard_trace=True):
    """Oracle results for ``streams`` with every decision clear of the guard.

    Mutates ``inp`` (seed[b] and possibly h[b]) for re-drawn streams and
    returns (results dict by stream, number of re-draws).
    """
    if streams is None:
        streams = range(int(inp["B"]))
    res, redraws = {}, 0
    for b in streams:
        b = int(b)
        for attempt in range(max_tries):
            r = dflash.cycle_stream(inp, b)
            bad = violations(r["margins"])
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
