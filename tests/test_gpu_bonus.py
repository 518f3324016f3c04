"""GPU parity where the drafts survive: long accept chains and the bonus token.

P1 "DFlash 2: Block diffusion, wearing a drafter's coat", "The architecture",
"Lossless, with conditions I did not used to state", and P3 "DFlash 2: Keep
Drafting Parallel", "What Happened": when the drafted path agrees with the
target, several tokens are kept per cycle and, once all L are kept, one more
is drawn from the target's row L+1.  The concurrent-32 inputs accept almost
nothing, so these inputs are built to accept:

* greedy (T = 0): zero embeddings and target rows 1..L equal to the drafter
  rows, so the greedy path is every position's drafter argmax, which is
  also the target argmax; every draft is accepted and the bonus is the
  argmax of row L+1;
* sampling (T > 0): one token of every drafter row raised by 30 and target
  rows 1..L equal to the drafter rows, so q and p both put nearly all their
  mass on it and every accept test passes (up to the guard's margin); row
  L+1 is left plain, so the bonus draw spreads over many chunks;
* every token a candidate (V = K), zero embeddings, target = drafter: q = p
  at every position.

Each input runs through dflash_cycle, the split entry points (dflash_topk,
dflash_pair_scores, dflash_trace, dflash_verify) and dflash_cycle_maxsum,
at L in {1, 8, 16} and mixed temperatures, against the oracle.
"""

import sys

import numpy as np
import pytest

import synth
from guard import guarded
from gpu_util import alloc_outputs, compare_stream, device_inputs, dims_of, run_cycle
from maxsum_util import guarded_maxsum, run_maxsum_fused, run_maxsum_split

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


GREEDY_ALL = dict(T=0.0, zero_E=True, noise=0.0, plant=None)
BOOSTED = dict(noise=0.0, plant=None, boost=30.0)

# (name, config id, overrides, every stream must accept all L drafts)
CASES = [
    ("T0-L1", 3, dict(B=4, L=1, V=20008, hidden=256, **GREEDY_ALL), True),
    ("T0-L8", 3, dict(B=4, V=20008, hidden=256, **GREEDY_ALL), True),
    ("T0-L16", 4, dict(B=3, V=20008, hidden=256, **GREEDY_ALL), True),
    ("mixedT-L1", 5, dict(B=6, L=1, V=12296, hidden=256, **BOOSTED), False),
    ("mixedT-L8", 5, dict(B=6, V=12296, hidden=256, **BOOSTED), False),
    ("mixedT-L16", 5, dict(B=6, L=16, V=12296, hidden=256, **BOOSTED), False),
    ("T1-L8-full-vocab", 3, dict(B=6, **BOOSTED), False),
    ("T06-V-eq-K", 3, dict(B=4, V=16, K=16, hidden=256, T=0.6, zero_E=True, noise=0.0, plant=None), False),
]


def _split_greedy(inp):
    import torch
    import block_draft_select_amd as dfl
    d = dims_of(inp)
    dev = device_inputs(inp)
    o = alloc_outputs(inp)
    ws = dfl.workspace(d)
    dfl.dflash_topk(d, dev["U"], o["cand_idx"], o["cand_logit"], ws)
    dfl.dflash_pair_scores(d, dev["x0"], o["cand_idx"], o["cand_logit"], dev["E"], dev["W"], dev["h"], o["S"], ws)
    dfl.dflash_trace(d, o["S"], o["cand_idx"], dev["T"], dev["seed"], inp["cycle"], o["path_rank"],
                     o["draft_tok"], o["q"])
    dfl.dflash_verify(d, dev["Z"], o["cand_idx"], o["path_rank"], o["q"], dev["T"], dev["seed"], inp["cycle"],
                      o["accept_len"], o["out_tok"], ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}


def _full_accepts(inp, res):
    L = int(inp["L"])
    greedy = sum(1 for b, r in res.items() if r["accept_len"] == L and not inp["T"][b] > 0)
    sampled = sum(1 for b, r in res.items() if r["accept_len"] == L and inp["T"][b] > 0)
    return greedy, sampled


@pytest.mark.parametrize("name,cid,kw,all_accept", CASES, ids=[c[0] for c in CASES])
def test_accept_chains_and_bonus(name, cid, kw, all_accept):
    inp = synth.make(cid, set_id=303, **kw)
    L, B = int(inp["L"]), int(inp["B"])
    _say(f"[bonus] {name}: B={B} L={L} V={inp['V']} K={inp['K']} T={sorted(set(map(float, inp['T'])))}")
    zero_e = bool(kw.get("zero_E"))
    ref, _ = guarded(inp, guard_trace=not zero_e)
    gpu = run_cycle(inp)
    for b in range(B):
        compare_stream(gpu, ref[b], b)
    split = _split_greedy(inp)
    for k, v in split.items():
        np.testing.assert_array_equal(v, gpu[k], err_msg=f"split vs cycle: {k}")
    g, s = _full_accepts(inp, ref)
    _say(f"[bonus] {name}: greedy cycle, streams accepting all {L}: {g} at T=0, {s} at T>0 (of {B})")
    if all_accept:
        assert g + s == B
    assert g + s >= 1

    ms_ref = guarded_maxsum(inp, range(B), guard_trace=not zero_e)
    ms_split = run_maxsum_split(inp)
    ms_fused = run_maxsum_fused(inp)
    for k, v in ms_split.items():
        np.testing.assert_array_equal(ms_fused[k], v, err_msg=f"max-sum fused vs split: {k}")
    for b in range(B):
        np.testing.assert_array_equal(ms_fused["path_rank"][b], ms_ref[b]["path_rank"], err_msg=f"path {b}")
        np.testing.assert_array_equal(ms_fused["draft_tok"][b], ms_ref[b]["draft_tok"], err_msg=f"draft {b}")
        assert int(ms_fused["accept_len"][b]) == int(ms_ref[b]["accept_len"]), f"accept_len {b}"
        np.testing.assert_array_equal(ms_fused["out_tok"][b], ms_ref[b]["out_tok"][: L + 1], err_msg=f"out {b}")
    g2, s2 = _full_accepts(inp, ms_ref)
    _say(f"[bonus] {name}: max-sum cycle, streams accepting all {L}: {g2} at T=0, {s2} at T>0 (of {B})")
    if all_accept:
        assert g2 + s2 == B


def test_bonus_reached_at_both_temperature_kinds():
    # the sampled cases above reach the bonus at T > 0 and the greedy cases
    # at T = 0: checked here on one small input of each kind, so that the
    # claim does not rest on the luck of the guard's redraws
    counts = {}
    for kw in (dict(B=6, V=12296, hidden=256, **BOOSTED),):
        inp = synth.make(5, set_id=304, **kw)
        ref, _ = guarded(inp)
        gpu = run_cycle(inp)
        for b in range(inp["B"]):
            compare_stream(gpu, ref[b], b)
        g, s = _full_accepts(inp, ref)
        counts["greedy"], counts["sampled"] = g, s
    _say(f"[bonus] streams reaching the bonus token: {counts}")
    assert counts["greedy"] >= 1 and counts["sampled"] >= 1
