"""The fused cycle replayed from a captured HIP graph.

A caller that captures dflash_cycle (with its own workspace) or
dflash_cycle_static (the library's static scratch, for callers that cannot
allocate) into a graph replays the same launches with the same arguments:
the cycle number is frozen, so every replay must give exactly the outputs
of an eager call with that cycle number, while the workspace's hand-off
epoch (device state, advanced by every cycle) keeps each replay's hand-off
entries apart from the previous cycle's.  Between replays the test runs
eager cycles of other inputs on the same workspace, so each replay meets
fresh entries of another cycle (P3 "DFlash 2: Keep Drafting Parallel",
"What Comes Next", paragraph "A Lightweight Path Selector": the candidate
lattice and its scores are rebuilt every cycle)."""

import sys

import numpy as np
import pytest

import synth
from gpu_util import alloc_outputs, device_inputs, dims_of, run_cycle

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


def _numpy(out):
    return {k: v.cpu().numpy() for k, v in out.items()}


def _same(a, b, what):
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), f"{what}: {k} differs from the eager call"


def _reset(out):
    # every output overwritten with a marker before a replay, so a replay
    # that skipped a write would be seen
    for v in out.values():
        v.fill_(float("nan") if v.dtype.is_floating_point else -7)


def _replays(call, between, inp, n_replay=4):
    """Capture call(out) into a graph; replay it n_replay times, each time
    checking every output against an eager call, with between() (eager
    work on the same workspace or scratch) after each replay."""
    import torch
    out_e = alloc_outputs(inp)
    call(out_e)
    torch.cuda.synchronize()
    ref = _numpy(out_e)
    out_g = alloc_outputs(inp)
    # warm-up on a side stream, then capture on torch's capture stream (the
    # binding launches on torch's current stream)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out_g)
    torch.cuda.synchronize()
    for rep in range(n_replay):
        _reset(out_g)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(ref, _numpy(out_g), f"replay {rep}")
        _say(f"[graph] replay {rep}: every output equals the eager call")
        between()
        torch.cuda.synchronize()


def _outputs_kw(out):
    return dict(cand_idx=out["cand_idx"], cand_logit=out["cand_logit"], S=out["S"],
                path_rank=out["path_rank"], draft_tok=out["draft_tok"], q=out["q"])


def test_cycle_with_workspace_replayed():
    import block_draft_select_amd as dfl
    inp = synth.make(3, set_id=31, B=4, V=20008, hidden=256)
    other = synth.make(3, set_id=32, B=4, V=20008, hidden=256)
    d = dims_of(inp)
    dev = device_inputs(inp)
    ws = dfl.workspace(d)

    def call(out):
        dfl.dflash_cycle(d, dev["U"], dev["Z"], dev["x0"], dev["E"], dev["W"], dev["h"], dev["T"], dev["seed"],
                         inp["cycle"], out["accept_len"], out["out_tok"], ws, **_outputs_kw(out))

    _say("[graph] dflash_cycle with a workspace")
    _replays(call, lambda: run_cycle(other, ws=ws), inp)


def test_static_cycle_replayed():
    # the static entry point's first call on the device (its symbol lookup)
    # is the eager reference call, outside the capture
    import block_draft_select_amd as dfl
    inp = synth.make(3, set_id=33, B=4, V=20008, hidden=256)
    other = synth.make(3, set_id=34, B=4, V=20008, hidden=256)
    d = dims_of(inp)
    dev, dev_o = device_inputs(inp), device_inputs(other)
    out_o = alloc_outputs(other)

    def call(out):
        dfl.dflash_cycle_static(d, dev["U"], dev["Z"], dev["x0"], dev["E"], dev["W"], dev["h"], dev["T"],
                                dev["seed"], inp["cycle"], out["accept_len"], out["out_tok"], **_outputs_kw(out))

    def between():
        # another cycle on the same static scratch
        dfl.dflash_cycle_static(d, dev_o["U"], dev_o["Z"], dev_o["x0"], dev_o["E"], dev_o["W"], dev_o["h"],
                                dev_o["T"], dev_o["seed"], other["cycle"], out_o["accept_len"], out_o["out_tok"])

    _say("[graph] dflash_cycle_static")
    _replays(call, between, inp)
