"""GPU parity of the two-tap convolution: the HIP path (``dflash_conv2tap``,
through the C ABI) against the float64 oracle (``oracle.conv``).

Bar: every output within (H + 4) * 2^-24 of its magnitude bound
sum_k |Wt[c, k] x_t[k]| * |x_t[c]| + sum_k |Wt[H + c, k] x_t[k]| * |x_{t-1}[c]|:
each tap is an fp32 sum of H products (exact for bf16 operands, one rounding
each for fp32 ones), then two products and one fused add.
"""

import sys

import numpy as np
import pytest

import synth
from gpu_util import _np_to_dev
from oracle import conv as C
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


def _run(inp):
    import torch
    import block_draft_select_amd as dfl
    B, L, H, pk = inp["B"], inp["L"], inp["hidden"], inp["param_kind"]
    d = dfl.dims(B, L, 64, 16, 16, H, "bf16", pk)
    x, x0, Wt = (_np_to_dev(inp[k], "cuda") for k in ("x", "x0", "Wt"))
    y = torch.full((B, L, H), float("nan"), dtype=torch.float32, device="cuda")
    dfl.dflash_conv2tap(d, x, x0, Wt, y)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def _check(inp, y, streams):
    H, pk = inp["hidden"], inp["param_kind"]
    x = O.widen(inp["x"], pk)
    x0 = O.widen(inp["x0"], pk)
    Wt = O.widen(inp["Wt"], pk)
    aW = np.abs(Wt)
    for b in streams:
        ref = C.conv2tap(x[b], x0[b], Wt)
        prev = np.vstack([x0[b][None], x[b][:-1]])
        ax = np.abs(x[b])
        taps_mag = ax @ aW.T                                   # [L, 2H]
        bound = taps_mag[:, :H] * ax + taps_mag[:, H:] * np.abs(prev)
        tol = (H + 4) * 2.0 ** -24 * bound + 1e-30
        err = np.abs(y[b] - ref)
        bad = np.argwhere(err > tol)
        assert bad.size == 0, (f"stream {b}: {len(bad)} outputs out of bound, first at {tuple(bad[0])}: "
                               f"gpu {y[b][tuple(bad[0])]!r} oracle {ref[tuple(bad[0])]!r} tol {tol[tuple(bad[0])]!r}")


CASES = [
    # (name, config id, overrides, streams compared (None: all))
    ("bf16-ragged", 3, dict(B=3, L=5, hidden=48), None),          # 15 rows, a half channel tile
    ("bf16-two-row-tiles", 3, dict(B=5, L=16, hidden=272), None),  # 80 rows, 17 channel tiles
    ("bf16-one-position", 3, dict(B=7, L=1, hidden=64), None),     # every row takes x0
    ("f32-small", 1, dict(B=2, L=3, hidden=32), None),
    ("f32-ragged", 1, dict(B=3, L=4, hidden=80), None),
    ("bf16-concurrent-32", 3, dict(), None),                       # B 32, L 8, hidden 2048
    ("bf16-large-vocab-128", 5, dict(), [0, 77, 127]),              # B 128, L 8, hidden 3072
    # limits: one row at the smallest hidden; a wide hidden on the small
    # tiles; the 128 x 64 tiles with ragged rows (500 = 3 * 128 + 116),
    # ragged channels (4112 = 64 * 64 + 16) and an odd stage count (one stage
    # of loads in flight)
    ("bf16-one-row-min-hidden", 3, dict(B=1, L=1, hidden=16), None),
    ("bf16-wide-hidden", 3, dict(B=2, L=2, hidden=4096), None),
    ("bf16-large-tiles-ragged", 3, dict(B=100, L=5, hidden=4112), [0, 51, 99]),
    # the 128 x 96 tiles (one block per CU, direct to LDS): ragged rows
    # (936 = 7 * 128 + 40), channels (2800 = 29 * 96 + 16) and k (2800 =
    # 43 * 64 + 48, the last stage cleared past the row end); then 960 rows
    # and 2944 channels (30 * 96 + 64) with whole stages
    ("bf16-wide-tiles-ragged", 3, dict(B=117, L=8, hidden=2800), [0, 58, 116]),
    ("bf16-wide-tiles-whole-stages", 3, dict(B=120, L=8, hidden=2944), [0, 119]),
    # the 128 x 64 tiles with two stages of loads in flight in registers
    ("bf16-large-tiles-two-stages", 3, dict(B=128, L=8, hidden=2048), [0, 64, 127]),
    # the smallest hidden on the large tilings (many rows): channel tiles
    # wider than hidden, one stage with a k tail; 32768 rows take the
    # 128 x 96 tiles, 40960 the 128 x 64 register-staged ones
    ("bf16-wide-tiles-min-hidden", 3, dict(B=2048, L=16, hidden=16), [0, 1023, 2047]),
    ("bf16-large-tiles-min-hidden", 3, dict(B=2560, L=16, hidden=16), [0, 1279, 2559]),
]


@pytest.mark.parametrize("name,cid,kw,streams", CASES, ids=[c[0] for c in CASES])
def test_conv2tap_matches_oracle(name, cid, kw, streams):
    inp = synth.make_conv(cid, set_id=4, **kw)
    _say(f"[conv] {name}: B={inp['B']} L={inp['L']} hidden={inp['hidden']} {inp['param_kind']}")
    y = _run(inp)
    assert np.isfinite(y).all()
    _check(inp, y, range(inp["B"]) if streams is None else streams)


def test_conv2tap_identity_generator_squares():
    # current taps = x_t, previous taps = 0 (a closed form on the GPU as well):
    # y = x * x, exact in fp32 for bf16 inputs
    inp = synth.make_conv(3, set_id=5, B=2, L=4, hidden=96)
    H = inp["hidden"]
    eye = np.vstack([np.eye(H, dtype=np.float32), np.zeros((H, H), dtype=np.float32)])
    inp["Wt"] = synth.bf16_bits(eye)
    y = _run(inp)
    x = O.widen(inp["x"], "bf16")
    np.testing.assert_array_equal(y, x * x)


@pytest.mark.parametrize("kw", [dict(B=4, L=8, hidden=256), dict(B=117, L=8, hidden=2800),
                                dict(B=128, L=8, hidden=2048)],
                         ids=["small-tiles", "wide-tiles", "register-ring"])
def test_conv2tap_graph_replay_equals_eager(kw):
    # the call enqueues one kernel and nothing else, so a caller may capture
    # it into a HIP graph; every replay must give the eager call's y exactly
    # (one tiling per case: 64 x 32 and 128 x 96 direct to LDS, 128 x 64
    # register-staged)
    import torch
    import block_draft_select_amd as dfl
    inp = synth.make_conv(3, set_id=6, **kw)
    B, L, H = inp["B"], inp["L"], inp["hidden"]
    _say(f"[conv] graph replay: B={B} L={L} hidden={H}")
    d = dfl.dims(B, L, 64, 16, 16, H, "bf16", "bf16")
    x, x0, Wt = (_np_to_dev(inp[k], "cuda") for k in ("x", "x0", "Wt"))
    y_ref = torch.empty((B, L, H), dtype=torch.float32, device="cuda")
    dfl.dflash_conv2tap(d, x, x0, Wt, y_ref)
    y = torch.empty_like(y_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dfl.dflash_conv2tap(d, x, x0, Wt, y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dfl.dflash_conv2tap(d, x, x0, Wt, y)
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep} differs from the eager call"
