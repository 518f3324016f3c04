"""GPU parity of the max-sum (Viterbi) trace: ``dflash_trace_viterbi`` through
the C ABI against the float64 oracle (``oracle.viterbi``), and the verify that
follows it against ``oracle.dflash.verify_stream`` with the one-hot q; the
fused ``dflash_cycle_maxsum`` must equal that split path bit for bit.

Bar: bit-exact path ranks, draft tokens, q (exactly one-hot), accept counts
and emitted tokens.  The GPU sums fp32 scores in fp64 and the oracle sums
fp64 scores, so inputs pass a margin guard first: every decision the oracle's
backtrack reads (and every accept/residual decision of the verify) must clear
the thresholds of ``tests/guard.py``; a stream that does not gets a fresh
context vector h (score gaps) or Philox seed (sampling decisions).
"""

import sys

import numpy as np
import pytest

import synth
from gpu_util import alloc_outputs, device_inputs, dims_of
from maxsum_util import guarded_maxsum as _guarded, run_maxsum_fused as _run_fused, run_maxsum_split as _run_split
from oracle import viterbi as VT

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_draft_select_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


CASES = [
    # (name, config id, overrides, streams compared (None: all))
    ("tiny-f32", 1, dict(B=3), None),
    ("strong-selector-T1", 3, dict(B=4, V=9000, hidden=256, e_std=0.3), None),
    ("strong-selector-T0", 2, dict(B=4, V=9000, hidden=256, e_std=0.3, T=0.0), None),
    ("strong-L16", 4, dict(B=3, V=20000, hidden=256, e_std=0.3), None),
    ("K4-L3", 3, dict(B=4, V=4096, hidden=256, K=4, L=3, e_std=0.3), None),
    ("K1-L1", 3, dict(B=2, V=1000, hidden=256, K=1, L=1), None),
    ("L2-mixedT", 5, dict(B=6, V=12296, hidden=512, L=2, e_std=0.3), None),
    ("concurrent-32", 3, dict(), [0, 13, 31]),
    # limits: every token a candidate (the residual has no chunk mass); the
    # largest row count B (L + 1) = 65535
    ("V-eq-K", 3, dict(B=3, V=16, K=16, hidden=256, plant=None, e_std=0.3), None),
    ("max-rows", 3, dict(B=3855, L=16, V=64, hidden=16, r=16, plant=None), [0, 1927, 3854]),
]


@pytest.mark.parametrize("name,cid,kw,streams", CASES, ids=[c[0] for c in CASES])
def test_viterbi_then_verify_match_oracle(name, cid, kw, streams):
    inp = synth.make(cid, set_id=211, **kw)
    streams = list(range(inp["B"])) if streams is None else streams
    _say(f"[viterbi] {name}: B={inp['B']} L={inp['L']} V={inp['V']} K={inp['K']}")
    ref = _guarded(inp, streams)
    gpu = _run_split(inp)
    fused = _run_fused(inp)
    for k, v in gpu.items():  # the fused max-sum cycle equals the split path bit for bit
        np.testing.assert_array_equal(fused[k], v, err_msg=f"fused vs split: {k}")
    L = int(inp["L"])
    for b in streams:
        np.testing.assert_array_equal(gpu["cand_idx"][b], ref[b]["cand_idx"], err_msg=f"cand_idx {b}")
        np.testing.assert_array_equal(gpu["path_rank"][b], ref[b]["path_rank"], err_msg=f"path_rank {b}")
        np.testing.assert_array_equal(gpu["draft_tok"][b], ref[b]["draft_tok"], err_msg=f"draft_tok {b}")
        np.testing.assert_array_equal(gpu["q"][b].astype(np.float64), ref[b]["q"], err_msg=f"q {b}")
        assert int(gpu["accept_len"][b]) == int(ref[b]["accept_len"]), f"accept_len {b}"
        np.testing.assert_array_equal(gpu["out_tok"][b], ref[b]["out_tok"][: L + 1], err_msg=f"out_tok {b}")


def test_viterbi_never_scores_below_greedy_on_gpu_scores():
    # on the GPU's own scores: the max-sum path's value is at least the
    # greedy trace's, and equal where the two paths coincide
    import torch
    import block_draft_select_amd as dfl
    inp = synth.make(3, set_id=212, B=8, V=9000, hidden=256, e_std=0.3, T=0.0)
    inp["T"][:] = 0.0
    d = dims_of(inp)
    dev = device_inputs(inp)
    o = alloc_outputs(inp)
    ws = dfl.workspace(d)
    dfl.dflash_topk(d, dev["U"], o["cand_idx"], o["cand_logit"], ws)
    dfl.dflash_pair_scores(d, dev["x0"], o["cand_idx"], o["cand_logit"], dev["E"], dev["W"], dev["h"], o["S"], ws)
    greedy = torch.empty_like(o["path_rank"])
    gtok = torch.empty_like(o["draft_tok"])
    gq = torch.empty_like(o["q"])
    dfl.dflash_trace(d, o["S"], o["cand_idx"], dev["T"], dev["seed"], 0, greedy, gtok, gq)
    dfl.dflash_trace_viterbi(d, o["S"], o["cand_idx"], o["path_rank"], o["draft_tok"], o["q"])
    torch.cuda.synchronize()
    S = o["S"].cpu().numpy().astype(np.float64)
    vp, gp = o["path_rank"].cpu().numpy(), greedy.cpu().numpy()
    differ = 0
    for b in range(inp["B"]):
        vv, gv = VT.path_value(S[b], vp[b]), VT.path_value(S[b], gp[b])
        assert vv >= gv - 1e-9 * max(1.0, abs(gv))
        differ += int((vp[b] != gp[b]).any())
    _say(f"[viterbi] streams whose max-sum path leaves the greedy one: {differ} of {inp['B']}")
