"""GPU parity of the acceptance-length study (``study_util``): on planted
lattices, every stream's accept count and emitted tokens under the four
selectors (independent top-1, the pair selector, the max-sum path, the
planted-path oracle selector), at T = 0 and T = 1, against the oracle."""

import sys

import numpy as np
import pytest

import synth
from study_util import SELECTORS, guard_subset, run_gpu, variant

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


@pytest.fixture(scope="module")
def lattice():
    return synth.make_lattice(7, B=24, V=16384, hidden=256)


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_study_selectors_match_oracle(lattice, T):
    import block_draft_select_amd as dfl
    from gpu_util import dims_of
    ws = dfl.workspace(dims_of(lattice))
    B, L = lattice["B"], lattice["L"]
    means = {}
    for sel in SELECTORS:
        x = variant(lattice, sel, T)
        ref = guard_subset(x, sel, range(B))
        acc, out = run_gpu(dfl, x, sel, ws)
        assert len(ref) >= B - 2, f"{sel}: {B - len(ref)} streams dropped as near-ties"
        for b, (n, o) in ref.items():
            assert int(acc[b]) == int(n), f"{sel} T={T} stream {b} accept_len"
            np.testing.assert_array_equal(out[b], o[: L + 1], err_msg=f"{sel} T={T} stream {b}")
        means[sel] = float(acc.mean())
        if sel == "top1":
            top1 = acc.copy()
        if sel == "oracle" and T == 0.0:
            # at T = 0 the oracle selector drafts the target's argmax wherever
            # the top-1 does, and more: never fewer accepted drafts
            assert np.all(acc >= top1)
    _say(f"[study] T={T}: mean accepted drafts " + ", ".join(f"{k} {v:.2f}" for k, v in means.items()))
