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


# ---------------------------------------------------------------- verify over a split

def _select(dfl, inp, dev, ws):
    """Candidates, path and q of the unsplit select half (dflash_topk,
    dflash_pair_scores, dflash_trace)."""
    from gpu_util import alloc_outputs, dims_of
    d = dims_of(inp)
    o = alloc_outputs(inp)
    dfl.dflash_topk(d, dev["U"], o["cand_idx"], o["cand_logit"], ws)
    dfl.dflash_pair_scores(d, dev["x0"], o["cand_idx"], o["cand_logit"], dev["E"], dev["W"], dev["h"], o["S"], ws)
    dfl.dflash_trace(d, o["S"], o["cand_idx"], dev["T"], dev["seed"], inp["cycle"], o["path_rank"],
                     o["draft_tok"], o["q"])
    return o


def _verify_shards(dfl, inp, dev, o, begins):
    """Per-shard statistics on each shard's own buffer, then the finalize
    over the split."""
    import torch
    from gpu_util import dims_of
    d = dims_of(inp)
    B, L, V = inp["B"], inp["L"], inp["V"]
    ends = begins[1:] + [V]
    shards = [dev["Z"][:, :, lo:hi].contiguous() for lo, hi in zip(begins, ends)]
    stats = torch.zeros(dfl.shard_stats_bytes(d, begins), dtype=torch.uint8, device="cuda")
    for s, zs in enumerate(shards):
        dfl.dflash_shard_stats(d, begins, s, zs, dev["T"], stats)
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, L + 1), -7, dtype=torch.int32, device="cuda")
    dfl.dflash_verify_shards(d, begins, shards, stats, o["cand_idx"], o["path_rank"], o["q"], dev["T"], dev["seed"],
                             inp["cycle"], acc, out)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy()


VERIFY_SPLITS = [
    # (name, config id, overrides, shard starts, streams compared (None: all))
    ("one-shard", 3, dict(B=4, V=20008, hidden=256), [0], None),
    ("two-ragged", 3, dict(B=4, V=20008, hidden=256), [0, 10000], None),
    ("three-ragged-mixedT", 5, dict(B=6, V=20008, hidden=256), [0, 6664, 13336], None),
    ("eight-of-151936", 3, dict(B=8, hidden=256), [i * 18992 for i in range(8)], None),
    ("eight-aligned-262144", 5, dict(B=6, hidden=256), [i * 32768 for i in range(8)], None),
    ("bonus-eight-ragged", 5, dict(B=6, V=20008, hidden=256, noise=0.0, plant=None, boost=30.0),
     [0, 2504, 5000, 7504, 10000, 12504, 15000, 17504], None),
    ("f32-three", 1, dict(B=3, V=4096, T=0.8), [0, 1364, 2732], None),
    ("concurrent-32-eight", 3, dict(), [i * 18992 for i in range(8)], [0, 11, 31]),
]


@pytest.mark.parametrize("name,cid,kw,begins,streams", VERIFY_SPLITS, ids=[c[0] for c in VERIFY_SPLITS])
def test_verify_over_a_vocabulary_split(name, cid, kw, begins, streams):
    import block_draft_select_amd as dfl
    from gpu_util import device_inputs, dims_of
    from guard import guarded
    inp = synth.make(cid, set_id=51, **kw)
    B, L, V = inp["B"], inp["L"], inp["V"]
    streams = list(range(B)) if streams is None else streams
    _say(f"[shard-verify] {name}: B={B} L={L} V={V} shards at {begins}")
    ref, redraws = guarded(inp, streams=streams, shard_begin=begins)
    dev = device_inputs(inp)
    ws = dfl.workspace(dims_of(inp))
    o = _select(dfl, inp, dev, ws)
    acc, out = _verify_shards(dfl, inp, dev, o, begins)
    ranks = o["path_rank"].cpu().numpy()
    for b in streams:
        np.testing.assert_array_equal(ranks[b], ref[b]["path_rank"], err_msg=f"path {b}")
        assert int(acc[b]) == int(ref[b]["accept_len"]), f"accept_len {b}"
        np.testing.assert_array_equal(out[b], ref[b]["out_tok"][: L + 1], err_msg=f"out_tok {b}")
    full = sum(int(ref[b]["accept_len"] == L) for b in streams)
    _say(f"[shard-verify] {name}: {len(streams)} streams equal the oracle ({redraws} redraws, {full} reach the bonus)")
    # a single shard, or boundaries on the chunk grid, give the unsplit
    # chunks: the outputs must then equal dflash_verify's bit for bit
    if all(b0 % 4096 == 0 for b0 in begins):
        import torch
        d = dims_of(inp)
        acc1 = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        out1 = torch.full((B, L + 1), -7, dtype=torch.int32, device="cuda")
        dfl.dflash_verify(d, dev["Z"], o["cand_idx"], o["path_rank"], o["q"], dev["T"], dev["seed"], inp["cycle"],
                          acc1, out1, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc1.cpu().numpy(), acc)
        np.testing.assert_array_equal(out1.cpu().numpy(), out)
