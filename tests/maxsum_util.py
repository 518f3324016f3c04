"""Helpers of the max-sum GPU tests: the oracle of the max-sum cycle (the
float64 max-sum path, then the verify with a one-hot q), its margin guard,
and the split and fused max-sum paths run through the C ABI."""

import numpy as np

from guard import _redraw_h, violations
from gpu_util import alloc_outputs, device_inputs, dims_of
from oracle import dflash as O
from oracle import viterbi as VT


def oracle_maxsum_stream(inp, b):
    r = O.cycle_stream(inp, b)
    path, draft, _, m = VT.viterbi_stream(r["S"], r["cand_idx"])
    L, K = int(inp["L"]), int(inp["K"])
    q = np.zeros((L, K))
    q[np.arange(L), path] = 1.0
    Zr = O.widen(inp["Z"][b], inp["logit_kind"])
    n, out, mv = O.verify_stream(Zr, r["cand_idx"], path, q, float(np.float32(inp["T"][b])), int(inp["seed"][b]),
                                 int(inp["cycle"]))
    return dict(cand_idx=r["cand_idx"], path_rank=path, draft_tok=draft, q=q, accept_len=n, out_tok=out), m + mv


def guarded_maxsum(inp, streams, max_tries=40, guard_trace=True):
    res = {}
    for b in streams:
        for attempt in range(max_tries):
            r, m = oracle_maxsum_stream(inp, b)
            bad = violations(m)
            if not guard_trace:
                bad = [x for x in bad if x[0] != "trace_gap"]
            if not bad:
                break
            if any(k == "trace_gap" for k, _, _ in bad):
                _redraw_h(inp, b, 100 + attempt)
            else:
                inp["seed"][b] = np.uint64((int(inp["seed"][b]) + (1 << 48) * (attempt + 1)) & 0xFFFFFFFFFFFFFFFF)
        else:
            raise RuntimeError(f"stream {b}: no guard-clean input")
        res[b] = r
    return res


def run_maxsum_split(inp):
    import torch
    import block_draft_select_amd as dfl
    d = dims_of(inp)
    dev = device_inputs(inp)
    o = alloc_outputs(inp)
    ws = dfl.workspace(d)
    dfl.dflash_topk(d, dev["U"], o["cand_idx"], o["cand_logit"], ws)
    dfl.dflash_pair_scores(d, dev["x0"], o["cand_idx"], o["cand_logit"], dev["E"], dev["W"], dev["h"], o["S"], ws)
    dfl.dflash_trace_viterbi(d, o["S"], o["cand_idx"], o["path_rank"], o["draft_tok"], o["q"])
    dfl.dflash_verify(d, dev["Z"], o["cand_idx"], o["path_rank"], o["q"], dev["T"], dev["seed"], inp["cycle"],
                      o["accept_len"], o["out_tok"], ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}


def run_maxsum_fused(inp):
    import torch
    import block_draft_select_amd as dfl
    d = dims_of(inp)
    dev = device_inputs(inp)
    o = alloc_outputs(inp)
    ws = dfl.workspace(d)
    dfl.dflash_cycle_maxsum(d, dev["U"], dev["Z"], dev["x0"], dev["E"], dev["W"], dev["h"], dev["T"], dev["seed"],
                            inp["cycle"], o["accept_len"], o["out_tok"], ws, cand_idx=o["cand_idx"],
                            cand_logit=o["cand_logit"], S=o["S"], path_rank=o["path_rank"],
                            draft_tok=o["draft_tok"], q=o["q"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}
