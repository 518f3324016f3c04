"""dflash_cycle_static (the cycle on the library's own static scratch, for
callers that cannot allocate) against dflash_cycle with a workspace: the
same outputs bit for bit, on two calls in a row, the second with a smaller
input, then a call beyond the static maximum that is rejected and leaves
its outputs untouched."""

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


def _run_static(inp):
    import torch
    import block_draft_select_amd as dfl
    d = dims_of(inp)
    dev = device_inputs(inp)
    o = alloc_outputs(inp)
    dfl.dflash_cycle_static(d, dev["U"], dev["Z"], dev["x0"], dev["E"], dev["W"], dev["h"], dev["T"], dev["seed"],
                            inp["cycle"], o["accept_len"], o["out_tok"], cand_idx=o["cand_idx"],
                            cand_logit=o["cand_logit"], S=o["S"], path_rank=o["path_rank"],
                            draft_tok=o["draft_tok"], q=o["q"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}


def test_static_scratch_cycle_equals_workspace_cycle():
    import block_draft_select_amd as dfl
    # concurrent-32 at full size (1.2 MiB of scratch), then a smaller,
    # mixed-temperature input: the second call must not see the first's
    # leftovers
    big = synth.make(3, set_id=41)
    small = synth.make(5, set_id=42, B=5, V=12296, hidden=256, boost=30.0, noise=0.0, plant=None)
    for inp in (big, small):
        need = dfl.workspace_bytes(dims_of(inp))
        _say(f"[static] B={inp['B']} L={inp['L']} V={inp['V']}: {need} bytes of scratch")
        assert need <= dfl.STATIC_SCRATCH_BYTES
        got = _run_static(inp)
        ref = run_cycle(inp)
        for k in ref:
            np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
        _say(f"[static] equal to dflash_cycle; accept_len {list(got['accept_len'][:8])}")


def test_static_scratch_rejects_oversize_and_launches_nothing():
    import torch
    import block_draft_select_amd as dfl
    inp = synth.make(3, set_id=43, B=3855, L=16, V=64, hidden=16, r=16, plant=None)
    d = dims_of(inp)
    dev = device_inputs(inp)
    o = alloc_outputs(inp)
    with pytest.raises(dfl.DFlashError) as e:
        dfl.dflash_cycle_static(d, dev["U"], dev["Z"], dev["x0"], dev["E"], dev["W"], dev["h"], dev["T"],
                                dev["seed"], 0, o["accept_len"], o["out_tok"])
    assert e.value.status == dfl.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(o["accept_len"] == -7) and torch.all(o["out_tok"] == -7)
