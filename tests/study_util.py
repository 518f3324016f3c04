"""Synthetic acceptance-length study: four ways of choosing the drafted path
on planted lattices (``synth.make_lattice``), run through the library and
checked against the oracle on a subset of streams.

P3 "DFlash 2: Keep Drafting Parallel", "What Comes Next": a selector that
always took the right candidate would lift the accepted length a lot, and
the lightweight pair selector recovers part of that gap at T = 0 and T = 1.
The four selectors:
  top1     the candidates' independent best (the pair term switched off:
           zero embeddings), greedy or sampled as the temperature says;
  selector the pair selector (dflash_cycle);
  maxsum   the max-sum path over the same scores (dflash_cycle_maxsum);
  oracle   the planted token whenever it is among the K candidates, the
           top candidate otherwise, with a one-hot q (dflash_topk, then
           dflash_verify on that path): an analysis device that knows the
           planted path, not a product path.
"""

import numpy as np

from guard import violations, score_sensitivity
from gpu_util import alloc_outputs, device_inputs, dims_of
from oracle import dflash as O
from oracle import viterbi as VT

SELECTORS = ("top1", "selector", "maxsum", "oracle")


def planted_path(cand_idx, planted):
    """Ranks of the oracle selector: the planted token's rank where it is a
    candidate, rank 0 elsewhere.  cand_idx [..., L, K], planted [..., L]."""
    hit = cand_idx == planted[..., None]
    return np.where(hit.any(-1), hit.argmax(-1), 0).astype(np.int32)


def variant(inp, selector, T):
    """The input set a selector runs on at temperature T (copies)."""
    x = dict(inp)
    x["T"] = np.full(inp["B"], T, dtype=np.float32)
    x["seed"] = inp["seed"].copy()
    if selector == "top1":
        x["E"] = np.zeros_like(inp["E"])
    return x


def oracle_stream(x, b, selector):
    """(accept_len, out_tok, margins, greedy-trace sensitivity) of one
    stream under a selector, from the float64 oracle."""
    r = O.cycle_stream(x, b)
    if selector in ("top1", "selector"):
        return r["accept_len"], r["out_tok"], r["margins"], score_sensitivity(r)
    L, K = int(x["L"]), int(x["K"])
    if selector == "maxsum":
        path, _, _, m = VT.viterbi_stream(r["S"], r["cand_idx"])
    else:
        path, m = planted_path(r["cand_idx"], x["planted"][b, :L]), []
    q = np.zeros((L, K))
    q[np.arange(L), path] = 1.0
    n, out, mv = O.verify_stream(O.widen(x["Z"][b], x["logit_kind"]), r["cand_idx"], path, q,
                                 float(np.float32(x["T"][b])), int(x["seed"][b]), int(x["cycle"]))
    return n, out, m + mv, None


def guard_subset(x, selector, streams, max_tries=20):
    """Oracle results of ``streams`` with every decision clear of the guard:
    a sampling decision too close to its boundary redraws the stream's seed
    in ``x``; a near-tie of scores (which only a new context would move)
    drops the stream from the subset.  Returns {stream: (n, out)}."""
    res = {}
    for b in streams:
        for attempt in range(max_tries):
            n, out, m, sens = oracle_stream(x, b, selector)
            bad = violations(m, sens)
            if not bad:
                res[b] = (n, out)
                break
            if any(k == "trace_gap" for k, _, _ in bad):
                break
            x["seed"][b] = np.uint64((int(x["seed"][b]) + (1 << 48) * (attempt + 1)) & 0xFFFFFFFFFFFFFFFF)
    return res


def run_gpu(dfl, x, selector, ws, dev=None):
    """accept_len [B] and out_tok [B, L+1] of one selector on the GPU."""
    import torch
    d = dims_of(x)
    dev = dev or device_inputs(x)
    o = alloc_outputs(x)
    if selector in ("top1", "selector"):
        dfl.dflash_cycle(d, dev["U"], dev["Z"], dev["x0"], dev["E"], dev["W"], dev["h"], dev["T"], dev["seed"],
                         x["cycle"], o["accept_len"], o["out_tok"], ws)
    elif selector == "maxsum":
        dfl.dflash_cycle_maxsum(d, dev["U"], dev["Z"], dev["x0"], dev["E"], dev["W"], dev["h"], dev["T"],
                                dev["seed"], x["cycle"], o["accept_len"], o["out_tok"], ws)
    else:
        dfl.dflash_topk(d, dev["U"], o["cand_idx"], o["cand_logit"], ws)
        torch.cuda.synchronize()
        L, K = int(x["L"]), int(x["K"])
        path = planted_path(o["cand_idx"].cpu().numpy(), x["planted"][:, :L])
        pr = torch.from_numpy(path).cuda()
        q = torch.nn.functional.one_hot(pr.long(), K).float().contiguous()
        dfl.dflash_verify(d, dev["Z"], o["cand_idx"], pr, q, dev["T"], dev["seed"], x["cycle"], o["accept_len"],
                          o["out_tok"], ws)
    torch.cuda.synchronize()
    return o["accept_len"].cpu().numpy(), o["out_tok"].cpu().numpy()
