"""Helpers for GPU tests: move synthetic inputs to the device and run the
library through its C ABI (via the package binding)."""

import numpy as np


def _np_to_dev(a, device):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.uint64:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int64)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def dims_of(inp):
    import block_draft_select_amd as dfl
    return dfl.dims(inp["B"], inp["L"], inp["V"], inp["K"], inp["r"], inp["hidden"],
                    inp["logit_kind"], inp["param_kind"])


def device_inputs(inp, device="cuda"):
    keys = ("U", "Z", "x0", "E", "W", "h", "T", "seed")
    return {k: _np_to_dev(inp[k], device) for k in keys}


def alloc_outputs(inp, device="cuda"):
    import torch
    B, L, K = inp["B"], inp["L"], inp["K"]
    i32 = dict(dtype=torch.int32, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    return dict(
        accept_len=torch.full((B,), -7, **i32), out_tok=torch.full((B, L + 1), -7, **i32),
        cand_idx=torch.full((B, L, K), -7, **i32), cand_logit=torch.full((B, L, K), np.nan, **f32),
        S=torch.full((B, L, K, K), np.nan, **f32), path_rank=torch.full((B, L), -7, **i32),
        draft_tok=torch.full((B, L), -7, **i32), q=torch.full((B, L, K), np.nan, **f32))


def run_cycle(inp, dev=None, out=None, ws=None, device="cuda"):
    """One dflash_cycle on `inp`; returns numpy copies of every output."""
    import torch
    import block_draft_select_amd as dfl
    d = dims_of(inp)
    dev = dev or device_inputs(inp, device)
    out = out or alloc_outputs(inp, device)
    ws = ws if ws is not None else dfl.workspace(d, device)
    dfl.dflash_cycle(d, dev["U"], dev["Z"], dev["x0"], dev["E"], dev["W"], dev["h"], dev["T"], dev["seed"],
                     inp["cycle"], out["accept_len"], out["out_tok"], ws,
                     cand_idx=out["cand_idx"], cand_logit=out["cand_logit"], S=out["S"],
                     path_rank=out["path_rank"], draft_tok=out["draft_tok"], q=out["q"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def q_tolerance(ref):
    """Per-entry bound on |q_gpu - q_ref| for one stream's sampled trace.

    q_t = softmax(S[t, prev, :] / T) is formed in fp64 on both sides, but
    from fp32 scores on the GPU: each score carries an absolute error of at
    most about 2^-23 max(1, |S row|), which moves log q_t(j) by at most twice
    that divided by T, so |dq| <= q * 2^-21 max(1, |S row|) / T with a
    factor two to spare; 2e-6 covers the fp32 rounding of q itself."""
    T, S, path = ref.get("T", 0.0), ref["S"], ref["path_rank"]
    q = ref["q"]
    tol = np.full(q.shape, 2e-6)
    if T > 0:
        prev = 0
        for t in range(q.shape[0]):
            tol[t] += q[t] * 2.0 ** -21 * max(1.0, float(np.abs(S[t, prev]).max())) / T
            prev = int(path[t])
    return tol


def compare_stream(gpu, ref, b, check_q=True):
    """Assert the parity bar for stream b: exact integers, scores within
    1e-4 relative (floor 1), q within the bound of ``q_tolerance``."""
    L = ref["cand_idx"].shape[0]
    np.testing.assert_array_equal(gpu["cand_idx"][b], ref["cand_idx"], err_msg=f"cand_idx stream {b}")
    np.testing.assert_array_equal(gpu["cand_logit"][b].astype(np.float64), ref["cand_val"],
                                  err_msg=f"cand_logit stream {b}")
    S_ref = ref["S"]
    tol = 1e-4 * np.maximum(1.0, np.abs(S_ref))
    assert np.all(np.abs(gpu["S"][b].astype(np.float64) - S_ref) <= tol), f"S stream {b}"
    np.testing.assert_array_equal(gpu["path_rank"][b], ref["path_rank"], err_msg=f"path_rank stream {b}")
    np.testing.assert_array_equal(gpu["draft_tok"][b], ref["draft_tok"], err_msg=f"draft_tok stream {b}")
    if check_q:
        assert np.all(np.abs(gpu["q"][b].astype(np.float64) - ref["q"]) <= q_tolerance(ref)), f"q stream {b}"
    assert int(gpu["accept_len"][b]) == int(ref["accept_len"]), f"accept_len stream {b}"
    np.testing.assert_array_equal(gpu["out_tok"][b], ref["out_tok"][: L + 1], err_msg=f"out_tok stream {b}")
