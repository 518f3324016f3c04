"""GPU parity of the two-launch cycle's hand-off inside the streaming launch.

The edge blocks read the top-K lists and gate partials of the same launch
as self-validating entries (a tag mixed from the workspace's cycle epoch,
a check word): stale entries of earlier cycles, entries of other shapes
and arbitrary workspace contents must never be taken for this cycle's.
Each case runs dflash_cycle on a workspace in such a state and compares
every stream with the oracle (P3 "DFlash 2: Keep Drafting Parallel",
"What Comes Next", paragraph "A Lightweight Path Selector": the pair
scores of candidates at neighbouring positions)."""

import sys

import numpy as np
import pytest

import synth
from guard import guarded
from gpu_util import compare_stream, dims_of, run_cycle

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


def _check(inp, ref, gpu, what):
    for b in ref:
        compare_stream(gpu, ref[b], b)
    _say(f"[handoff] {what}: {len(ref)} streams equal the oracle")


def test_random_workspace_contents():
    # a workspace full of random bytes (not zero-filled) before the first
    # cycle: every entry of the hand-off regions is garbage
    import torch
    import block_draft_select_amd as dfl
    inp = synth.make(3, set_id=11, B=6, V=20008, hidden=256)
    ref, _ = guarded(inp)
    d = dims_of(inp)
    g = torch.Generator(device="cuda").manual_seed(1234)
    ws = torch.randint(0, 256, (max(dfl.workspace_bytes(d), 16),), dtype=torch.uint8, device="cuda", generator=g)
    _say("[handoff] random workspace")
    _check(inp, ref, run_cycle(inp, ws=ws), "random workspace, first cycle")
    _check(inp, ref, run_cycle(inp, ws=ws), "random workspace, second cycle")


def test_shapes_alternating_on_one_workspace():
    # two shapes (both in the two-launch form) take turns on one workspace
    # sized for the larger: each cycle meets the other shape's entries
    import block_draft_select_amd as dfl
    a = synth.make(3, set_id=12, B=4, V=20008, hidden=256)
    b = synth.make(5, set_id=13, B=6, L=5, V=12296, hidden=512)
    ref_a, _ = guarded(a)
    ref_b, _ = guarded(b)
    ws = dfl.workspace(dims_of(b)) if dfl.workspace_bytes(dims_of(b)) > dfl.workspace_bytes(dims_of(a)) \
        else dfl.workspace(dims_of(a))
    _say("[handoff] alternating shapes")
    for rep in range(3):
        _check(a, ref_a, run_cycle(a, ws=ws), f"shape A, turn {rep}")
        _check(b, ref_b, run_cycle(b, ws=ws), f"shape B, turn {rep}")


def test_split_calls_between_cycles():
    # the split entry points use the same workspace between two cycles
    import torch
    import block_draft_select_amd as dfl
    from gpu_util import alloc_outputs, device_inputs
    a = synth.make(3, set_id=14, B=4, V=20008, hidden=256)
    b = synth.make(3, set_id=15, B=4, V=20008, hidden=256)
    ref_a, _ = guarded(a)
    d = dims_of(a)
    ws = dfl.workspace(d)
    _check(a, ref_a, run_cycle(a, ws=ws), "cycle before split calls")
    dev = device_inputs(b)
    o = alloc_outputs(b)
    dfl.dflash_topk(d, dev["U"], o["cand_idx"], o["cand_logit"], ws)
    dfl.dflash_pair_scores(d, dev["x0"], o["cand_idx"], o["cand_logit"], dev["E"], dev["W"], dev["h"], o["S"], ws)
    torch.cuda.synchronize()
    r = run_cycle(a, ws=ws)
    _check(a, ref_a, r, "cycle after split calls")
    np.testing.assert_array_equal(r["out_tok"], run_cycle(a, ws=ws)["out_tok"])
