"""GPU parity: the HIP path against the float64 oracle, through the C ABI.

Bar: bit-exact candidate indices and logits, selected paths, draft tokens,
accept counts and emitted tokens; pair scores within 1e-4 relative (floor 1);
q within 2e-6 absolute.  Inputs are seeded synthetic sets (``synth``) passed
through the oracle's near-tie margin guard (``tests/guard.py``).
"""

import sys

import numpy as np
import pytest

import synth
from guard import guarded
from gpu_util import alloc_outputs, compare_stream, device_inputs, dims_of, run_cycle

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


# (name, config id, overrides, guard the greedy trace gap)
SMALL = [
    ("tiny-f32-greedy", 1, dict(), True),
    ("tiny-f32-sampling", 1, dict(B=3, T=0.8), True),
    ("bf16-T1-ragged", 3, dict(B=4, V=20008, hidden=256), True),
    ("bf16-T0-ragged", 2, dict(B=3, V=20008, hidden=256), True),
    ("bf16-mixedT", 5, dict(B=6, V=12296, hidden=512), True),
    ("bf16-strong-selector", 3, dict(B=4, V=9000, hidden=256, e_std=0.3), True),
    ("bf16-strong-greedy", 2, dict(B=3, V=9000, hidden=256, e_std=0.3, T=0.0), True),
    ("bf16-ties-T1", 3, dict(B=3, V=16392, hidden=256, ties=True), True),
    ("bf16-ties-T0", 2, dict(B=3, V=16392, hidden=256, ties=True, T=0.0), True),
    ("bf16-K4-L3", 3, dict(B=4, V=4096, hidden=256, K=4, L=3), True),
    ("bf16-K1-L1", 3, dict(B=2, V=1000, hidden=256, K=1, L=1), True),
    ("bf16-L16", 4, dict(B=2, V=20000, hidden=256), True),
    ("bf16-r16-T06", 3, dict(B=3, V=8200, hidden=64, r=16, T=0.6), True),
    ("bf16-single-chunk", 3, dict(B=5, V=64, K=16, hidden=256, plant=None), True),
    # large logits at a low temperature: the chunk sums must not lose the
    # terms near each chunk's maximum to the rounding of m / T
    ("bf16-T01-logits35", 3, dict(B=4, V=20008, hidden=256, T=0.1, shift=35.0), True),
    ("bf16-T06-logits-40", 5, dict(B=6, V=12296, hidden=256, T=0.6, shift=-40.0), True),
    # temperatures that are not positive (0, negative, -0, NaN) are greedy
    ("bf16-nonpositive-T", 5, dict(B=6, V=12296, hidden=256,
                                   T=[0.0, -1.0, float("nan"), 0.6, -0.0, 1.0]), True),
]


@pytest.mark.parametrize("name,cid,kw,gt", SMALL, ids=[c[0] for c in SMALL])
def test_cycle_matches_oracle_small(name, cid, kw, gt):
    inp = synth.make(cid, set_id=101, **kw)
    _say(f"[parity] {name}: B={inp['B']} L={inp['L']} V={inp['V']} K={inp['K']} r={inp['r']}")
    ref, redraws = guarded(inp, guard_trace=gt)
    gpu = run_cycle(inp)
    for b in range(inp["B"]):
        compare_stream(gpu, ref[b], b)


# more seeded input sets of three representative shapes: sampling at T = 1
# with a ragged vocabulary, mixed temperatures, a strong selector whose paths
# leave top-1
SEEDS = [(cid, kw, sid) for cid, kw in (
    (3, dict(B=4, V=20008, hidden=256)),
    (5, dict(B=6, V=12296, hidden=512)),
    (3, dict(B=4, V=9000, hidden=256, e_std=0.3)),
) for sid in (102, 103, 104, 105)]


@pytest.mark.parametrize("cid,kw,sid", SEEDS, ids=[f"c{c[0]}-V{c[1]['V']}-set{c[2]}" for c in SEEDS])
def test_cycle_matches_oracle_more_sets(cid, kw, sid):
    inp = synth.make(cid, set_id=sid, **kw)
    _say(f"[parity] set {sid}: config {cid} B={inp['B']} V={inp['V']}")
    ref, _ = guarded(inp)
    gpu = run_cycle(inp)
    for b in range(inp["B"]):
        compare_stream(gpu, ref[b], b)


@pytest.mark.parametrize("ties", [False, True])
def test_zero_embeddings_independent_top1(ties):
    inp = synth.make(3, set_id=5, B=4, V=8192, hidden=256, zero_E=True, ties=ties, T=0.0)
    _say(f"[parity] zero-E ties={ties}")
    ref, _ = guarded(inp, guard_trace=False)
    gpu = run_cycle(inp)
    assert np.all(gpu["path_rank"] == 0)
    for b in range(inp["B"]):
        compare_stream(gpu, ref[b], b)


# the five configurations at full size, every stream compared (the largest
# in two halves, so that each test stays short; the halves share one input
# set, whose redrawn seeds stay guard-clean for the streams already checked)
FULL = [
    ("C1", 1, None),
    ("C2", 2, None),
    ("C3", 3, None),
    ("C4", 4, None),
    ("C5-first-half", 5, range(0, 64)),
    ("C5-second-half", 5, range(64, 128)),
]
_FULL_INPUTS = {}


@pytest.mark.parametrize("name,cid,streams", FULL, ids=[c[0] for c in FULL])
def test_full_size_configs_every_stream(name, cid, streams):
    if cid not in _FULL_INPUTS:
        _FULL_INPUTS.clear()
        _FULL_INPUTS[cid] = synth.make(cid, set_id=0)
    inp = _FULL_INPUTS[cid]
    streams = list(range(inp["B"]) if streams is None else streams)
    _say(f"[parity] full {name}: B={inp['B']} L={inp['L']} V={inp['V']} streams {streams[0]}..{streams[-1]}")
    ref, redraws = guarded(inp, streams=streams)
    gpu = run_cycle(inp)
    for b in ref:
        compare_stream(gpu, ref[b], b)
    L = int(inp["L"])
    full = sum(int(r["accept_len"] == L) for r in ref.values())
    acc = sum(int(r["accept_len"]) for r in ref.values())
    _say(f"[parity] full {name}: {len(ref)} streams equal the oracle; {redraws} guard redraws; "
         f"accepted drafts {acc}; streams accepting all {L}: {full}")


# block sizes the serving runtimes use (blocks of 4 to 16 drafted
# positions) at the concurrent-32 shapes, on sampled streams
BLOCKS = [4, 5, 7]


@pytest.mark.parametrize("L", BLOCKS, ids=[f"L{L}" for L in BLOCKS])
def test_block_size_sweep_sampled(L):
    inp = synth.make(3, set_id=0, L=L)
    streams = [0, 17, 31]
    _say(f"[parity] block sweep: B={inp['B']} L={inp['L']} V={inp['V']} streams={streams}")
    ref, _ = guarded(inp, streams=streams)
    gpu = run_cycle(inp)
    for b in ref:
        compare_stream(gpu, ref[b], b)


# limits of the boundary: every token a candidate (the residual has no
# chunk mass), the largest vocabulary (more chunk terms than the finalize
# keeps in LDS), and the largest row count B (L + 1) = 65535
EXTREME = [
    ("bf16-V-eq-K", 3, dict(B=3, V=16, K=16, hidden=256, plant=None), None),
    ("f32-V-eq-K4", 1, dict(B=2, V=4, K=4, T=0.8), None),
    ("bf16-max-V", 3, dict(B=1, L=4, V=2097152, hidden=256, plant=None), None),
    # one stream of a 151936-token vocabulary: ten partial lists per row
    ("bf16-ten-lists-T0", 2, dict(B=1, V=151936, hidden=256), None),
    ("bf16-ten-lists-T1", 3, dict(B=1, V=151936, hidden=256), None),
    ("bf16-max-rows", 3, dict(B=3855, L=16, V=64, hidden=16, r=16, plant=None), [0, 1, 1927, 3854]),
]


@pytest.mark.parametrize("name,cid,kw,streams", EXTREME, ids=[c[0] for c in EXTREME])
def test_extreme_shapes(name, cid, kw, streams):
    inp = synth.make(cid, set_id=9, **kw)
    _say(f"[parity] extreme {name}: B={inp['B']} L={inp['L']} V={inp['V']} K={inp['K']}")
    ref, _ = guarded(inp, streams=streams)
    gpu = run_cycle(inp)
    for b in ref:
        compare_stream(gpu, ref[b], b)


def test_all_nan_target_row_stays_in_range():
    # a greedy target row whose every logit is NaN has no argmax (the
    # results are unspecified) but the call must succeed and every emitted
    # token stay in range; the other stream is unaffected
    inp = synth.make(2, set_id=8, B=2, V=12296, hidden=256, T=0.0)
    _say("[parity] all-NaN target row")
    ref, _ = guarded(inp, streams=[0], guard_trace=False)
    inp["Z"][1, 0] = 0x7FC0
    inp["Z"][1, 2] = 0x7FC0
    gpu = run_cycle(inp)
    compare_stream(gpu, ref[0], 0)
    V, L = inp["V"], inp["L"]
    assert 0 <= gpu["accept_len"][1] <= L
    n = int(gpu["accept_len"][1])
    assert np.all((gpu["out_tok"][1][: n + 1] >= 0) & (gpu["out_tok"][1][: n + 1] < V))
    assert np.all(gpu["out_tok"][1][n + 1:] == -1)


def test_rows_without_admissible_values_stay_in_range():
    # a drafter row made only of the all-ones NaN pattern has no admissible
    # value, so its top lists stay empty; the cycle must still keep every
    # index it gathers and writes in range (the other stream is unaffected)
    inp = synth.make(3, set_id=6, B=2, V=8192, hidden=256)
    _say("[parity] empty candidate lists")
    ref, _ = guarded(inp, streams=[0])
    inp["U"][1] = 0xFFFF
    gpu = run_cycle(inp)
    compare_stream(gpu, ref[0], 0)
    V, L = inp["V"], inp["L"]
    assert np.all((gpu["cand_idx"][1] >= 0) & (gpu["cand_idx"][1] < V))
    assert 0 <= gpu["accept_len"][1] <= L
    assert np.all((gpu["out_tok"][1] >= -1) & (gpu["out_tok"][1] < V))
    assert np.all((gpu["path_rank"][1] >= 0) & (gpu["path_rank"][1] < inp["K"]))


def test_split_entry_points_equal_cycle():
    import torch
    import block_draft_select_amd as dfl
    inp = synth.make(3, set_id=77, B=3, V=20008, hidden=256)
    _say("[parity] split entry points vs dflash_cycle")
    d = dims_of(inp)
    dev = device_inputs(inp)
    whole = run_cycle(inp, dev=dev)
    o = alloc_outputs(inp)
    ws = dfl.workspace(d)
    dfl.dflash_topk(d, dev["U"], o["cand_idx"], o["cand_logit"], ws)
    dfl.dflash_pair_scores(d, dev["x0"], o["cand_idx"], o["cand_logit"], dev["E"], dev["W"], dev["h"], o["S"], ws)
    dfl.dflash_trace(d, o["S"], o["cand_idx"], dev["T"], dev["seed"], inp["cycle"], o["path_rank"],
                     o["draft_tok"], o["q"])
    dfl.dflash_verify(d, dev["Z"], o["cand_idx"], o["path_rank"], o["q"], dev["T"], dev["seed"], inp["cycle"],
                      o["accept_len"], o["out_tok"], ws)
    torch.cuda.synchronize()
    for k, v in o.items():
        np.testing.assert_array_equal(v.cpu().numpy(), whole[k], err_msg=k)


def test_deterministic_and_workspace_reuse():
    import block_draft_select_amd as dfl
    a = synth.make(5, set_id=3, B=5, V=12296, hidden=256)
    b = synth.make(5, set_id=4, B=5, V=12296, hidden=256)
    _say("[parity] determinism + workspace reuse")
    ref_a, _ = guarded(a)
    ref_b, _ = guarded(b)
    ws = dfl.workspace(dims_of(a))
    r1 = run_cycle(a, ws=ws)
    r2 = run_cycle(b, ws=ws)
    r3 = run_cycle(a, ws=ws)
    for k in r1:
        np.testing.assert_array_equal(r1[k], r3[k], err_msg=k)
    for s in range(a["B"]):
        compare_stream(r1, ref_a[s], s)
        compare_stream(r2, ref_b[s], s)


def test_topk_alone_special_rows():
    import torch
    import block_draft_select_amd as dfl
    from oracle import dflash as O
    _say("[parity] topk special rows")
    V, K, L = 16392, 16, 8
    rng = np.random.default_rng(3)
    rows = np.zeros((L, V), dtype=np.float32)
    rows[0] = 1.5                                           # all equal: lowest 16 indices
    rows[1] = -3.0
    rows[1, 5000:5010] = -0.0                              # signed zeros among negatives
    rows[1, 7000:7010] = 0.0
    rows[2] = np.sort(rng.standard_normal(V))[::-1]         # descending: concentrated in few lanes
    rows[3] = np.sort(rng.standard_normal(V))               # ascending: top at the ragged tail
    rows[4] = np.round(rng.standard_normal(V) * 2) / 2      # heavy ties
    rows[5] = rng.standard_normal(V) * 1e-3 - 50.0           # all negative
    # equal maxima scattered through every 4096-value block: about 100 per
    # block (more candidates than one per lane) and about 300 (more than
    # the candidate buffer holds)
    for t_, n_ in ((6, 100), (7, 300)):
        rows[t_] = -1.0
        for b0 in range(0, V, 4096):
            pos = rng.choice(np.arange(b0, min(b0 + 4096, V)), size=min(n_, V - b0), replace=False)
            rows[t_, pos] = 2.0
    bits = synth.bf16_bits(rows)
    inp = dict(B=1, L=L, V=V, K=K, r=16, hidden=16, logit_kind="bf16", param_kind="bf16")
    d = dims_of(inp)
    U = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    ci = torch.empty((L, K), dtype=torch.int32, device="cuda")
    cl = torch.empty((L, K), dtype=torch.float32, device="cuda")
    dfl.dflash_topk(d, U, ci, cl, dfl.workspace(d))
    torch.cuda.synchronize()
    for t in range(L):
        idx, val = O.topk_row(O.widen(bits[t], "bf16"), K)
        np.testing.assert_array_equal(ci[t].cpu().numpy(), idx, err_msg=f"row {t}")
        np.testing.assert_array_equal(cl[t].cpu().numpy().astype(np.float64), val, err_msg=f"row {t}")


def test_invalid_calls_launch_nothing():
    import torch
    import block_draft_select_amd as dfl
    _say("[parity] invalid calls")
    inp = synth.make(3, set_id=1, B=2, V=4096, hidden=256)
    d = dims_of(inp)
    dev = device_inputs(inp)
    o = alloc_outputs(inp)
    small = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(dfl.DFlashError) as e:
        dfl.dflash_cycle(d, dev["U"], dev["Z"], dev["x0"], dev["E"], dev["W"], dev["h"], dev["T"], dev["seed"],
                         0, o["accept_len"], o["out_tok"], small)
    assert e.value.status == dfl.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(o["accept_len"] == -7) and torch.all(o["out_tok"] == -7)
