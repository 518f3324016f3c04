"""GPU parity of the top-K over a vocabulary split: every shard runs
``dflash_topk`` on its own contiguous [B, L, width] slice of the drafter
logits, and ``dflash_topk_merge`` combines the shards' lists.  The result
must equal ``dflash_topk`` over the whole vocabulary bit for bit (indices
and values), and the oracle's top-K.
"""

import sys

import numpy as np
import pytest

import synth
from gpu_util import _np_to_dev
from oracle import dflash as O

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


def _topk(dfl, inp, U, V):
    import torch
    B, L, K = inp["B"], inp["L"], inp["K"]
    d = dfl.dims(B, L, V, K, inp["r"], inp["hidden"], inp["logit_kind"], inp["param_kind"])
    ci = torch.full((B, L, K), -7, dtype=torch.int32, device="cuda")
    cv = torch.full((B, L, K), float("nan"), dtype=torch.float32, device="cuda")
    dfl.dflash_topk(d, U, ci, cv, dfl.workspace(d))
    return ci, cv


SPLITS = [
    # (name, config id, overrides, shard starts as fractions of V rounded to 8, rows checked against the oracle)
    ("two-even", 3, dict(B=4), [0, 0.5], [(0, 0), (3, 7)]),
    ("eight-even", 3, dict(B=4), [i / 8 for i in range(8)], [(1, 2), (2, 5)]),
    ("five-ragged", 3, dict(B=4), [0, 0.03, 0.41, 0.42, 0.9], [(0, 3), (3, 0)]),
    ("f32-three", 1, dict(B=3, V=4096), [0, 0.25, 0.6], [(0, 0), (2, 7)]),
    ("one-shard", 3, dict(B=2, V=20008), [0], [(1, 4)]),
]


@pytest.mark.parametrize("name,cid,kw,fracs,rows", SPLITS, ids=[c[0] for c in SPLITS])
def test_sharded_topk_equals_whole(name, cid, kw, fracs, rows):
    import torch
    import block_draft_select_amd as dfl
    inp = synth.make(cid, set_id=41, **kw)
    B, L, V, K = inp["B"], inp["L"], inp["V"], inp["K"]
    begins = sorted({int(f * V) // 8 * 8 for f in fracs})
    _say(f"[shard] {name}: B={B} L={L} V={V} shards at {begins}")
    U = _np_to_dev(inp["U"], "cuda")
    whole_i, whole_v = _topk(dfl, inp, U, V)
    ends = begins[1:] + [V]
    parts_i, parts_v = [], []
    for lo, hi in zip(begins, ends):
        Us = U[:, :, lo:hi].contiguous()  # the shard's own buffer
        pi, pv = _topk(dfl, inp, Us, hi - lo)
        parts_i.append(pi)
        parts_v.append(pv)
    idx_parts = torch.stack(parts_i).contiguous()
    val_parts = torch.stack(parts_v).contiguous()
    d = dfl.dims(B, L, V, K, inp["r"], inp["hidden"], inp["logit_kind"], inp["param_kind"])
    mi = torch.full((B, L, K), -7, dtype=torch.int32, device="cuda")
    mv = torch.full((B, L, K), float("nan"), dtype=torch.float32, device="cuda")
    dfl.dflash_topk_merge(d, begins, idx_parts, val_parts, mi, mv)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(mi.cpu().numpy(), whole_i.cpu().numpy())
    np.testing.assert_array_equal(mv.cpu().numpy().view(np.uint32), whole_v.cpu().numpy().view(np.uint32))
    Uw = O.widen(inp["U"], inp["logit_kind"])
    for b, t in rows:
        ref_i, ref_v = O.topk_row(Uw[b, t], K)
        np.testing.assert_array_equal(mi[b, t].cpu().numpy(), ref_i)
        np.testing.assert_array_equal(mv[b, t].cpu().numpy().astype(np.float64), ref_v)
