#!/usr/bin/env python3
"""Throughput of the DFlash 2 draft -> select -> verify cycle on one MI355X.

One step = one dflash_cycle call (top-K over the drafter rows, gate, pair
scores, trace, target-row statistics and verify) for a whole batch of
streams, with every input already resident in HBM.  Input sets rotate so
that the timed working set exceeds twice the 256 MB last-level cache.

Prints one JSON line:
  value      draft-verify cycles/s on one GPU
  roofline   achieved algorithmic GB/s of the dominant kernel vs 8 TB/s
  cpu_baseline  the float64 NumPy oracle on a bounded sample, host cores
"""

import argparse
import glob
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "draft-verify cycles/s + logit HBM GB/s (% of peak) at B=32, L=8, V=151936"
HBM_PEAK_GBPS = 8000.0
LLC_BYTES = 256 << 20


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "block_draft_select_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def logit_bytes(inp):
    s = 2 if inp["logit_kind"] == "bf16" else 4
    u = inp["B"] * inp["L"] * inp["V"] * s
    z = inp["B"] * (inp["L"] + 1) * inp["V"] * s
    return u, z


def workload_name(inp):
    Ts = sorted(set(float(t) for t in inp["T"]))
    return (f"{inp['name']}: B={inp['B']} L={inp['L']} V={inp['V']} K={inp['K']} r={inp['r']} "
            f"hidden={inp['hidden']} logits={inp['logit_kind']} params={inp['param_kind']} T={Ts}")


_POOL_INPUT = None


def _oracle_stream(b):
    """One stream of the oracle in a worker process (single-threaded BLAS)."""
    import threadpoolctl
    from oracle import dflash as O
    with threadpoolctl.threadpool_limits(1):
        O.cycle_stream(_POOL_INPUT, b)
    return b


def cpu_baseline(inp, seconds, max_workers=16):
    """The oracle as it stands on the host's cores, on a bounded sample.

    The streams of a cycle are independent, so whole cycles run with one
    stream per task over a pool of worker processes (forked before this
    process touches the GPU, at most 16: the host share of one GPU), each
    single-threaded; the median of the timed cycles gives `value`.  The
    single-core rate (a bounded run of consecutive streams in this process)
    is reported beside it.
    """
    global _POOL_INPUT
    import multiprocessing as mp
    import threadpoolctl
    from oracle import dflash as O
    B = inp["B"]
    done, t0 = 0, time.perf_counter()
    with threadpoolctl.threadpool_limits(1):
        while done < B and (time.perf_counter() - t0) < seconds / 2:
            O.cycle_stream(inp, done)
            done += 1
    el1 = time.perf_counter() - t0
    single = {"value": 1.0 / (el1 / done * B), "cores": 1,
              "sample": f"{done} of {B} streams of input set 0 ({el1:.1f} s), scaled to one {B}-stream cycle"}
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    workers = max(1, min(max_workers, affinity, B))
    _POOL_INPUT = inp
    times = []
    with mp.get_context("fork").Pool(workers) as pool:
        pool.map(_oracle_stream, range(min(B, workers)))  # workers started and warm
        t_all = time.perf_counter()
        while len(times) < 3 or (time.perf_counter() - t_all) < seconds / 2:
            t1 = time.perf_counter()
            pool.map(_oracle_stream, range(B), chunksize=1)
            times.append(time.perf_counter() - t1)
            if time.perf_counter() - t_all > seconds and len(times) >= 1:
                break
    _POOL_INPUT = None
    times.sort()
    med = times[len(times) // 2]
    cpu = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": 1.0 / med, "unit": "cycles/s", "cores": workers, "kind": "oracle",
            "sample": f"{len(times)} whole {B}-stream cycles of input set 0, one stream per task over "
                      f"{workers} single-threaded worker processes (median {med:.2f} s per cycle)",
            "single_core": single,
            "host_cpu": cpu, "host_cpu_count": os.cpu_count(), "host_affinity": affinity}


def load_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary.

    The summary (profiles/traffic_<kernel>_<workload>.txt, "key: value"
    lines) holds FETCH_SIZE + WRITE_SIZE of the kernel scaled by what the
    same counters read for a plain copy of known size.  It counts only
    while the kernel sources are the ones it was taken on.
    """
    tag = workload.split(":", 1)[0].replace("-", "")
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{tag}.txt")
    if not os.path.exists(p):
        return None
    kv = {}
    with open(p) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "#", "|")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha") != kernel_source_sha():
        return None
    try:
        return int(float(kv["bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense bf16 MFMA; fp32 vector (the fp32 path's VALU)


def conv_leg(args, base, dfl):
    """The two-tap convolution at this workload's block shape [B, L, hidden].

    Generator matrices rotate across enough sets that they stream from HBM
    rather than from the last-level cache (set 0 from the seeded generator,
    the others drawn on the device with the same distribution).  The kernel
    duration comes from the library's per-launch timer.  Its roofline is the
    larger of two floors: the algorithmic bytes (x, x0 and Wt read once, y
    written once) at 8 TB/s and the GEMM's 2 * (B*L) * hidden * (2*hidden)
    flops at the matrix-core peak of the parameter type.
    """
    import torch
    import synth
    from gpu_util import _np_to_dev
    B, L, H, pk = base["B"], base["L"], base["hidden"], base["param_kind"]
    ps = 2 if pk == "bf16" else 4
    R = B * L
    wt_bytes = 2 * H * H * ps
    n_sets = max(1, min(64, -(-2 * LLC_BYTES // wt_bytes)))
    c0 = synth.make_conv(base["config_id"], set_id=0, B=B, L=L, hidden=H)
    sets = [{k: _np_to_dev(c0[k], "cuda") for k in ("x", "x0", "Wt")}]
    tdt = torch.bfloat16 if pk == "bf16" else torch.float32
    for _ in range(1, n_sets):
        sets.append({"x": torch.randn(B, L, H, device="cuda").to(tdt),
                     "x0": torch.randn(B, H, device="cuda").to(tdt),
                     "Wt": (torch.randn(2 * H, H, device="cuda") * 0.02).to(tdt)})
    y = torch.empty(B, L, H, dtype=torch.float32, device="cuda")
    d = dfl.dims(B, L, 64, 16, 16, H, "bf16", pk)
    for i in range(max(args.warmup, n_sets)):
        s = sets[i % n_sets]
        dfl.dflash_conv2tap(d, s["x"], s["x0"], s["Wt"], y)
    torch.cuda.synchronize()
    # wall clock per call with the timer off (its events cost host time),
    # then the kernel durations with it on
    t0 = time.perf_counter()
    for i in range(args.conv_steps):
        s = sets[i % n_sets]
        dfl.dflash_conv2tap(d, s["x"], s["x0"], s["Wt"], y)
    torch.cuda.synchronize()
    wall_us = (time.perf_counter() - t0) * 1e6 / args.conv_steps
    dfl.dflash_profile_enable(True)
    for i in range(args.conv_steps):
        s = sets[i % n_sets]
        dfl.dflash_conv2tap(d, s["x"], s["x0"], s["Wt"], y)
    torch.cuda.synchronize()
    n, ms = dfl.dflash_profile_collect("conv2tap")
    dfl.dflash_profile_enable(False)
    avg_us = ms * 1e3 / n
    nbytes = (R * H + B * H) * ps + wt_bytes + R * H * 4
    flops = 2.0 * R * H * 2 * H
    t_hbm = nbytes / (HBM_PEAK_GBPS * 1e9)
    t_mma = flops / (MFMA_PEAK_TFLOPS[pk] * 1e12)
    if t_hbm >= t_mma:
        roof = {"bound": "hbm", "achieved": round(nbytes / (avg_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(t_hbm / (avg_us * 1e-6), 4)}
    else:
        roof = {"bound": "mfma" if pk == "bf16" else "alu",
                "achieved": round(flops / (avg_us * 1e-6) / 1e12, 1), "peak": MFMA_PEAK_TFLOPS[pk],
                "unit": "TFLOP/s", "frac": round(t_mma / (avg_us * 1e-6), 4)}
    roof.update({"algorithmic_bytes_per_launch": nbytes, "flops_per_launch": flops,
                 "traffic": load_traffic("conv2tap", base["name"])})
    _log(f"[bench] conv2tap {avg_us:.2f} us/launch ({roof['frac']:.2f} of its {roof['bound']} roof)")
    return {"shape": f"B={B} L={L} hidden={H} {pk}", "launches": n, "avg_us": round(avg_us, 2),
            "wall_us_per_call": round(wall_us, 2), "generator_sets": n_sets, "roofline": roof}


def viterbi_leg(args, base, dfl, dv, d, ws):
    """The max-sum trace on input set 0's pair scores (computed once by the
    split entry points), timed per launch with the library's timer.  It is
    latency-bound: its bytes are the scores and candidate indices in, the
    path, draft tokens and one-hot q out."""
    import torch
    from gpu_util import alloc_outputs
    o = alloc_outputs(base)
    dfl.dflash_topk(d, dv["U"], o["cand_idx"], o["cand_logit"], ws)
    dfl.dflash_pair_scores(d, dv["x0"], o["cand_idx"], o["cand_logit"], dv["E"], dv["W"], dv["h"], o["S"], ws)
    for _ in range(args.warmup):
        dfl.dflash_trace_viterbi(d, o["S"], o["cand_idx"], o["path_rank"], o["draft_tok"], o["q"])
    torch.cuda.synchronize()
    dfl.dflash_profile_enable(True)
    for _ in range(args.viterbi_steps):
        dfl.dflash_trace_viterbi(d, o["S"], o["cand_idx"], o["path_rank"], o["draft_tok"], o["q"])
    torch.cuda.synchronize()
    n, ms = dfl.dflash_profile_collect("trace_viterbi")
    dfl.dflash_profile_enable(False)
    B, L, K = base["B"], base["L"], base["K"]
    nbytes = B * L * K * K * 4 + B * L * K * 4 + B * L * (2 + K) * 4
    avg_us = ms * 1e3 / n
    _log(f"[bench] trace_viterbi {avg_us:.2f} us/launch")
    return {"launches": n, "avg_us": round(avg_us, 2), "bytes_per_launch": nbytes, "bound": "latency",
            "note": "one wave per stream: L dependent max-plus steps over K x K scores"}


def split_leg(args, base, dfl, devs, d, ws):
    """The order a serving engine must call the path in: the select half
    (dflash_topk, dflash_pair_scores, dflash_trace) before the target's
    forward pass, the verify half (dflash_verify) after it.  Each half is
    timed on its own over the rotating input sets (wall clock between two
    synchronisations), and every launch with the library's per-launch timer;
    the streaming launches get their roofline from their algorithmic bytes
    (the drafter logits for the top-K, the target logits for the
    statistics)."""
    import torch
    from gpu_util import alloc_outputs
    o = alloc_outputs(base)
    n_sets = len(devs)

    def select(i):
        dv = devs[i % n_sets]
        dfl.dflash_topk(d, dv["U"], o["cand_idx"], o["cand_logit"], ws)
        dfl.dflash_pair_scores(d, dv["x0"], o["cand_idx"], o["cand_logit"], dv["E"], dv["W"], dv["h"], o["S"], ws)
        dfl.dflash_trace(d, o["S"], o["cand_idx"], dv["T"], dv["seed"], i, o["path_rank"], o["draft_tok"], o["q"])

    def verify(i):
        dv = devs[i % n_sets]
        dfl.dflash_verify(d, dv["Z"], o["cand_idx"], o["path_rank"], o["q"], dv["T"], dv["seed"], i,
                          o["accept_len"], o["out_tok"], ws)

    res = {}
    for name, fn in (("select_half", select), ("verify_half", verify)):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.split_steps):
            fn(args.warmup + i)
        torch.cuda.synchronize()
        res[name] = {"us_per_call": round((time.perf_counter() - t0) * 1e6 / args.split_steps, 2)}
    dfl.dflash_profile_enable(True)
    for i in range(args.profile_steps):
        select(i)
        verify(i)
    torch.cuda.synchronize()
    kern = {}
    for name in ("topk", "gate", "scores", "trace", "stats", "finalize"):
        n, ms = dfl.dflash_profile_collect(name)
        if n:
            kern[name] = round(ms * 1e3 / n, 2)
    dfl.dflash_profile_enable(False)
    ub, zb = logit_bytes(base)
    ps = 2 if base["param_kind"] == "bf16" else 4
    gate_bytes = (base["B"] * base["L"] + base["r"]) * base["hidden"] * ps
    algo = {"topk": ub, "stats": zb, "gate": gate_bytes}
    roof = {}
    for k, nbytes in algo.items():
        if k in kern:
            gbps = nbytes / (kern[k] * 1e-6) / 1e9
            roof[k] = {"bound": "hbm", "algorithmic_bytes": nbytes, "achieved": round(gbps, 1),
                       "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    res.update({"kernel_avg_us": kern, "roofline": roof,
                "note": "topk = both launches of dflash_topk (partial lists, then the per-row merge)"})
    _log(f"[bench] split path: select {res['select_half']['us_per_call']} us, verify "
         f"{res['verify_half']['us_per_call']} us; kernels " + ", ".join(f"{k}={v}us" for k, v in kern.items()))
    return res


def study_leg(args, dfl):
    """Synthetic acceptance-length study (tests/study_util.py): mean accepted
    drafts per cycle of four path selectors on planted lattices at T = 0 and
    T = 1, every selector run through the library on all streams, and the
    first streams of each run checked against the oracle."""
    import numpy as np
    import torch
    import synth
    from gpu_util import device_inputs, dims_of, _np_to_dev
    from study_util import SELECTORS, guard_subset, run_gpu, variant
    t0 = time.perf_counter()
    inp = synth.make_lattice(0, B=args.study_streams, V=args.study_vocab, hidden=256)
    B, L = inp["B"], inp["L"]
    ws = dfl.workspace(dims_of(inp))
    dev0 = device_inputs(inp)
    zero_E = torch.zeros_like(dev0["E"])
    subset = list(range(min(args.study_check, B)))
    out_rec, checked, equal, dropped = {}, 0, 0, 0
    for T in (0.0, 1.0):
        row = {}
        for sel in SELECTORS:
            x = variant(inp, sel, T)
            ref = guard_subset(x, sel, subset)
            dropped += len(subset) - len(ref)
            dev = dict(dev0, T=_np_to_dev(x["T"], "cuda"), seed=_np_to_dev(x["seed"], "cuda"),
                       E=zero_E if sel == "top1" else dev0["E"])
            acc, out = run_gpu(dfl, x, sel, ws, dev)
            for b, (n, o) in ref.items():
                checked += 1
                equal += int(int(acc[b]) == int(n) and np.array_equal(out[b], o[: L + 1]))
            row[sel] = {"mean_accepted": round(float(acc.mean()), 3),
                        "stderr": round(float(acc.std(ddof=1) / np.sqrt(B)), 3),
                        "tokens_per_cycle": round(float(acc.mean()) + 1.0, 3)}
        out_rec[f"T={T:g}"] = row
    el = time.perf_counter() - t0
    _log("[bench] study " + "; ".join(f"{k}: " + ", ".join(f"{s} {v['mean_accepted']:.2f}" for s, v in r.items())
                                       for k, r in out_rec.items()) + f" ({checked} oracle checks, {equal} equal)")
    return {"workload": f"planted lattices: B={B} streams, L={L}, V={inp['V']}, K={inp['K']}, r={inp['r']}, "
                        f"hidden=256, bf16; drafter rows x4, target mode on the planted token (p=0.8 at T=1), "
                        f"planted tokens share one embedding direction per stream (norm 2.8)",
            "selectors": list(SELECTORS), "results": out_rec,
            "oracle_check": {"streams_checked": checked, "equal": equal, "dropped_near_ties": dropped},
            "seconds": round(el, 1)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, help="input configuration id (1..5)")
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0: enough for 2x LLC)")
    ap.add_argument("--L", type=int, default=0, help="drafted positions per block (0: the configuration's)")
    ap.add_argument("--B", type=int, default=0,
                    help="streams (0: the configuration's); B/N is one GPU's share when streams shard over N GPUs")
    ap.add_argument("--V", type=int, default=0,
                    help="vocabulary (0: the configuration's); V/N is one GPU's share when the vocabulary shards "
                         "over N GPUs")
    ap.add_argument("--profile-steps", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="plain copies of a logit-sized buffer first (calibrates hardware byte counters)")
    ap.add_argument("--read-probe", type=int, default=3,
                    help="timed passes (after one warm-up pass) of a one-pass nontemporal read over every "
                         "input set's logits (read ceiling)")
    ap.add_argument("--conv-steps", type=int, default=200,
                    help="timed launches of the two-tap convolution at the workload's block shape (0: skip)")
    ap.add_argument("--split-steps", type=int, default=200,
                    help="timed calls of each half of the split entry points (0: skip)")
    ap.add_argument("--study-streams", type=int, default=256,
                    help="streams of the acceptance-length study on planted lattices (0: skip)")
    ap.add_argument("--study-vocab", type=int, default=32768, help="vocabulary of the study's lattices")
    ap.add_argument("--study-check", type=int, default=8,
                    help="streams of each study run checked against the oracle")
    ap.add_argument("--graph-cycles", type=int, default=20,
                    help="cycles captured into one HIP graph for the replay leg (0: skip)")
    ap.add_argument("--viterbi-steps", type=int, default=200,
                    help="timed launches of the max-sum trace on the workload's pair scores (0: skip)")
    args = ap.parse_args()

    if args.gpus != 1:
        sys.exit(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
                 "(the batch of streams would shard by stream across GPUs, with no exchange)")

    import torch
    import synth
    import block_draft_select_amd as dfl
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import alloc_outputs, device_inputs, dims_of

    t_gen = time.perf_counter()
    kw = {k: v for k, v in (("L", args.L), ("B", args.B), ("V", args.V)) if v}
    base = synth.make(args.config, set_id=0, **kw)
    # the CPU baseline first: its worker processes fork before this process
    # touches the GPU
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(base, args.cpu_seconds)
        _log(f"[bench] cpu baseline {cpu['value']:.4f} cycles/s on {cpu['cores']} cores "
             f"({cpu['single_core']['value']:.4f} on one)")
    torch.cuda.set_device(0)
    ub, zb = logit_bytes(base)
    n_sets = args.sets or max(1, min(64, -(-2 * LLC_BYTES // (ub + zb))))
    sets = [base] + [synth.make(args.config, set_id=s, plant=None, **kw) for s in range(1, n_sets)]
    devs = [device_inputs(s) for s in sets]
    _log(f"[bench] {workload_name(base)}; {n_sets} input sets generated in {time.perf_counter() - t_gen:.1f} s")

    d = dims_of(base)
    ws = dfl.workspace(d)
    out = alloc_outputs(base)

    if args.copy_probe:
        src = torch.ones(ub + zb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.copy_probe):
            dfl.dflash_copy_probe(dst, src)
        torch.cuda.synchronize()
        _log(f"[bench] {args.copy_probe} copies of {ub + zb} bytes done")
        del src, dst

    def step(i):
        dv = devs[i % n_sets]
        dfl.dflash_cycle(d, dv["U"], dv["Z"], dv["x0"], dv["E"], dv["W"], dv["h"], dv["T"], dv["seed"], i,
                         out["accept_len"], out["out_tok"], ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    _log(f"[bench] warmup {args.warmup} done")

    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    cycles_per_s = args.steps / elapsed
    mean_accept = float(out["accept_len"].float().mean().item())
    _log(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/cycle")

    # distribution of the cycle time: an event between consecutive cycles on
    # the launching stream (a separate loop, so `value` stays a plain
    # wall-clock throughput)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for i in range(args.steps):
        step(args.warmup + args.steps + i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps))
    pct = lambda f: per[min(len(per) - 1, int(f * (len(per) - 1) + 0.5))]
    cycle_us = {"p10": round(pct(0.1), 2), "median": round(pct(0.5), 2), "p90": round(pct(0.9), 2)}
    _log(f"[bench] cycle time p10/median/p90 {cycle_us['p10']}/{cycle_us['median']}/{cycle_us['p90']} us")

    # the same cycles replayed from a captured HIP graph: graph_cycles
    # consecutive cycles over the rotating sets captured once, the graph
    # replayed; the launches are the eager path's, but a replay repeats the
    # captured cycle numbers, so this times the launch path only (the
    # draws repeat) and `value` stays the eager rate
    graph = None
    if args.graph_cycles:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(args.graph_cycles):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(args.graph_cycles):
                step(i)
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // args.graph_cycles)
        tg = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        g_us = (time.perf_counter() - tg) * 1e6 / (reps * args.graph_cycles)
        graph = {"us_per_cycle": round(g_us, 2), "cycles_per_s": round(1e6 / g_us, 1),
                 "cycles_per_graph": args.graph_cycles, "replays": reps,
                 "note": "launch path only: a replay repeats the captured cycle numbers"}
        del g
        _log(f"[bench] graph replay {g_us:.1f} us/cycle ({args.graph_cycles} cycles per graph)")

    # per-kernel durations: HIP events recorded by the library around each
    # launch on the stream it launches on
    dfl.dflash_profile_enable(True)
    for i in range(args.profile_steps):
        step(i)
    torch.cuda.synchronize()
    kern = {}
    for name in dfl.KERNELS:
        n, ms = dfl.dflash_profile_collect(name)
        if n:
            kern[name] = {"launches": n, "avg_us": ms * 1e3 / n}
    dfl.dflash_profile_enable(False)
    _log("[bench] kernels " + ", ".join(f"{k}={v['avg_us']:.1f}us" for k, v in kern.items()))

    # one-pass nontemporal read of the same buffers, back to back (a pass
    # covers every input set's logits between two events): the measured
    # read ceiling of the streaming launch's access shape
    read_gbps = None
    if args.read_probe:
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        evs, nbytes = [], 0
        for p in range(args.read_probe + 1):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for dv in devs:
                for buf in (dv["U"], dv["Z"]):
                    dfl.dflash_read_probe(buf, sink)
            e1.record()
            if p:  # the first pass warms up
                evs.append((e0, e1))
                nbytes += sum(dv[k].numel() * dv[k].element_size() for dv in devs for k in ("U", "Z"))
        torch.cuda.synchronize()
        if evs:
            read_gbps = nbytes / (sum(a.elapsed_time(b) for a, b in evs) * 1e-3) / 1e9
            _log(f"[bench] read ceiling {read_gbps:.1f} GB/s")

    # algorithmic bytes of each launch: the streaming launch reads every
    # drafter and target logit once and the gate's inputs h [B, L, hidden]
    # and W_g [r, hidden] once; the pair scores read the embedding rows of
    # each stream's distinct lattice tokens (x0 and the L K candidates) once
    ps = 2 if base["param_kind"] == "bf16" else 4
    gate_bytes = (base["B"] * base["L"] + base["r"]) * base["hidden"] * ps
    emb_bytes = base["B"] * (base["L"] * base["K"] + 1) * base["r"] * ps
    algo = {"cycle_stream": ub + zb + gate_bytes, "cycle_scores": emb_bytes}
    if "cycle_scores" not in kern:
        # the two-launch cycle: the candidate/score work (and its embedding
        # reads) runs inside the streaming launch
        algo = {"cycle_stream": ub + zb + gate_bytes + emb_bytes}
    dom = "cycle_stream"  # the HBM-bound launch
    achieved = algo[dom] / (kern[dom]["avg_us"] * 1e-6) / 1e9 if dom in kern else None
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1) if achieved else None,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4) if achieved else None,
            "traffic": load_traffic(dom, base["name"]), "algorithmic_bytes_per_launch": algo[dom],
            "cycle_launches": 3 if "cycle_scores" in kern else 2}
    per_kernel_roof = {k: round(algo[k] / (kern[k]["avg_us"] * 1e-6) / 1e9, 1) for k in algo if k in kern}

    conv = conv_leg(args, base, dfl) if args.conv_steps else None
    viterbi = viterbi_leg(args, base, dfl, devs[0], d, ws) if args.viterbi_steps else None
    maxsum = None
    if args.viterbi_steps:
        # the whole cycle with the max-sum trace, same rotating inputs
        def step_maxsum(i):
            dv = devs[i % n_sets]
            dfl.dflash_cycle_maxsum(d, dv["U"], dv["Z"], dv["x0"], dv["E"], dv["W"], dv["h"], dv["T"], dv["seed"],
                                    i, out["accept_len"], out["out_tok"], ws)
        for i in range(args.warmup):
            step_maxsum(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(args.steps):
            step_maxsum(args.warmup + i)
        torch.cuda.synchronize()
        el = time.perf_counter() - t1
        maxsum = {"value": round(args.steps / el, 2), "unit": "cycles/s",
                  "us_per_cycle": round(el * 1e6 / args.steps, 2)}
        _log(f"[bench] max-sum cycle {maxsum['us_per_cycle']:.1f} us/cycle")

    split = split_leg(args, base, dfl, devs, d, ws) if args.split_steps else None
    study = study_leg(args, dfl) if args.study_streams else None

    logit_gbps = (ub + zb) / (ms_per_step * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(cycles_per_s, 2),
        "unit": "cycles/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "cycle_us": cycle_us,
        "graph_replay": graph,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": workload_name(base), "B": base["B"], "L": base["L"], "V": base["V"],
                   "K": base["K"], "r": base["r"], "hidden": base["hidden"], "input_sets": n_sets},
        "logit_GBps": round(logit_gbps, 1),
        "logit_frac_of_peak": round(logit_gbps / HBM_PEAK_GBPS, 4),
        "roofline": roof,
        "kernel_GBps": per_kernel_roof,
        "read_ceiling_GBps": round(read_gbps, 1) if read_gbps else None,
        "frac_of_read_ceiling": round(achieved / read_gbps, 4) if (read_gbps and achieved) else None,
        "kernel_avg_us": {k: round(v["avg_us"], 2) for k, v in kern.items()},
        "mean_accept_len": round(mean_accept, 3),
        "conv2tap": conv,
        "trace_viterbi": viterbi,
        "cycle_maxsum": maxsum,
        "split_path": split,
        "acceptance_study": study,
        "cpu_baseline": cpu,
        "kernel_source_sha": kernel_source_sha(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
