#!/usr/bin/env python3
"""Throughput of the speculative-decoding verify step (libspecverify) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4]

One step is one full verify call on one batch of seeded synthetic logits that
already sit in HBM: for a chain workload ``sv_chain_verify`` (row statistics,
then accept / first rejection / residual-or-bonus resample / emit); for ``c5``
``sv_tree_verify_greedy`` (one launch for its 27-node trees: row argmax, with
each tree walked by the wave of its last chunk).  ``R`` copies of the inputs (at least 1 GiB in all,
four times the 256 MB Infinity Cache) are rotated so that every step reads HBM.

Prints one JSON line.  ``roofline`` rates the dominant kernel (the chain's
row-statistics kernel; the greedy call's one launch) on its algorithmic bytes,
2 * V * bytes_per_logit per drafted position (V * bytes_per_logit per tree
row), over its median duration in a leg of ``--kernel-reps`` full calls (100
by default, independent of ``--steps``) run after the timed steps, the chain
through its two stage calls.  Each duration comes from HIP events attached to
the launch itself (``sv_chain_row_stats_timed`` / ``sv_tree_verify_greedy_timed``
/ ``sv_chain_verify_ex``): the dispatch's own begin and end timestamps, the
interval rocprofv3's kernel trace reports.  For the greedy call,
``argmax_only`` times the two-launch form's row-argmax kernel (the same
stream without the walks) beside it.  ``mass_kernel`` does the same for
the chain's accept / resample kernel, on the bytes of the rows it samples from
(two rows per rejecting request, the bonus row otherwise).  ``traffic`` comes from the
rocprofv3 FETCH_SIZE / WRITE_SIZE summary under ``profiles/`` when it was taken
on the current kernel source, else null.
``cpu_baseline`` times the fp64 oracle on the same host arrays.

``--copy-calibration`` instead runs a plain 1 GiB device copy (the reference
kernel for scaling the FETCH_SIZE / WRITE_SIZE counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified draft positions/sec + achieved HBM GB/s (% of peak) at V=128256 bf16"
UNIT = "verified positions/s"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
POOL_CAP = 16                  # oracle worker processes at most
ROTATE_BYTES = 1 << 30
_CSRC = "sampling_spec_verify_amd/csrc/"
KERNEL_SOURCES = {
    "row_stats": [_CSRC + "sv_chain.hip", _CSRC + "sv_device.hpp", _CSRC + "sv_common.hpp"],
    "row_argmax": [_CSRC + "sv_tree.hip", _CSRC + "sv_device.hpp", _CSRC + "sv_common.hpp"],
    "greedy_fold": [_CSRC + "sv_tree.hip", _CSRC + "sv_device.hpp", _CSRC + "sv_common.hpp"],
}
COUNTER_FILE = os.path.join(ROOT, "profiles", "counters_{kernel}_{workload}.md")


def kernel_source_hash(kernel: str = "row_stats") -> str:
    """Hash of the sources the named kernel is built from."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if still current."""
    path = COUNTER_FILE.format(kernel=kernel, workload=workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    start = text.find("```json")
    if start < 0:
        return None
    end = text.find("```", start + 7)
    rec = json.loads(text[start + 7:end])
    if rec.get("kernel_source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("traffic_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="c4",
                    choices=["c1", "c2", "c3", "c4", "c5", "c5path", "c5mask", "c5multi"])
    ap.add_argument("--alpha", action="store_true",
                    help="chain workloads: time the acceptance-rate call instead of the verify call")
    ap.add_argument("--space", default="prob", choices=["prob", "logit"],
                    help="chain workloads: mix the two models in probability space (the "
                         "mixture equation) or logit space (the pseudocode's form)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound on the oracle's CPU time for cpu_baseline (0 disables)")
    ap.add_argument("--time-every", type=int, default=0,
                    help="also attach timing events to the dominant kernel of every n-th timed "
                         "step (0: none; the roofline comes from the --kernel-reps leg)")
    ap.add_argument("--kernel-reps", type=int, default=100,
                    help="launch-attached timings of the dominant kernel (and of the chain's "
                         "accept / resample kernel) in a leg of their own after the timed steps; "
                         "the roofline uses their median")
    ap.add_argument("--cpu-pool-seconds", type=float, default=6.0,
                    help="bound on the all-cores oracle run (a fork pool over requests, taken "
                         "before the GPU is touched); 0 disables")
    ap.add_argument("--graph", type=int, default=0, metavar="REPLAYS",
                    help="chain, greedy tree and mask workloads: also time REPLAYS replays of a "
                         "HIP graph holding one call per rotated buffer set (64 mask calls) - "
                         "the steady state without host launch gaps")
    ap.add_argument("--no-stream-ceiling", action="store_true",
                    help="skip the same-run read-stream ceiling measurement")
    ap.add_argument("--copy-calibration", action="store_true")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 5}), flush=True)


def device_copies(arr, dtype, R, torch):
    import numpy as np
    host = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16) if dtype == "bf16" else arr)
    base = host.to("cuda:0")
    if dtype == "bf16":
        base = base.view(torch.bfloat16)
    return [base] + [base.clone() for _ in range(R - 1)]


def read_stream_ceiling(nbytes, torch, sv, launches=60):
    """Same-run practical read ceiling: ``sv_read_stream`` (the row streams' access
    pattern, no arithmetic) over ``nbytes`` with buffer sets rotated past 1 GiB, and
    over one 2 GiB buffer.  Launch-attached events, as for the verify kernels."""
    import numpy as np

    def timed(views, n, k):
        sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        for i in range(5):
            sv.read_stream(views[i % len(views)], n, sink)
        timer = sv.KernelTimer(k)
        for i in range(k):
            sv.read_stream(views[i % len(views)], n, sink, timer.pair(i))
        torch.cuda.synchronize()
        ms = np.array([timer.elapsed_ms(i) for i in range(k)])
        timer.close()
        return ms

    stride = (nbytes + 4095) // 4096 * 4096
    R = max(2, math.ceil(ROTATE_BYTES / stride))
    buf = torch.empty(R * stride, dtype=torch.uint8, device="cuda:0")
    ms = timed([buf[i * stride:(i + 1) * stride] for i in range(R)], nbytes, launches)
    del buf
    big_n = 2 << 30
    big = torch.empty(big_n, dtype=torch.uint8, device="cuda:0")
    ms2 = timed([big], big_n, 20)
    del big
    torch.cuda.empty_cache()
    med, med2 = float(np.median(ms)), float(np.median(ms2))
    return {"kernel": "sv_read_stream", "bytes": nbytes, "buffer_sets_rotated": R,
            "launches": launches, "ms_median": med, "gbs_median": nbytes / (med * 1e-3) / 1e9,
            "gbs_2gib_median": big_n / (med2 * 1e-3) / 1e9}


_POOL = {}


def _pool_chain_worker(wid, nworkers, seconds):
    import oracle
    x, space, t, d = _POOL["x"], _POOL["space"], _POOL["t"], _POOL["d"]
    lens = x.lengths()
    done = pos = 0
    t0 = time.perf_counter()
    b = wid % x.B
    while time.perf_counter() - t0 < seconds:
        k = int(lens[b])
        oracle.chain_verify_one(t[b, :k + 1], d[b, :k], x.tokens[b, :k], x.u_accept[b, :k],
                                x.u_sample[b], x.lam, x.temperature, space)
        pos += k
        done += 1
        b = (b + nworkers) % x.B
    return done, pos


def _pool_tree_worker(wid, nworkers, seconds):
    import oracle
    x, t = _POOL["x"], _POOL["t"]
    done = 0
    t0 = time.perf_counter()
    b = wid % x.B
    while time.perf_counter() - t0 < seconds:
        oracle.tree_greedy_one(t[b], x.parent[b], x.node_token[b])
        done += 1
        b = (b + nworkers) % x.B
    return done, done * x.N


def cpu_pool_baseline(x, tree, seconds, space="prob", cores=None):
    """The oracle on all of the host's cores: one forked worker per core (at most 16),
    each cycling over its share of the batch's requests for ``seconds``.  Called before
    anything touches the GPU, so the workers are plain copies of a CPU-only process."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    host = len(os.sched_getaffinity(0))
    n = max(1, min(POOL_CAP, host)) if cores is None else cores
    # widened once here, as in the one-core run; the workers share the arrays
    _POOL.update(x=x, space=space, t=x.widened(x.target),
                 d=None if tree else x.widened(x.draft))
    fn = _pool_tree_worker if tree else _pool_chain_worker
    t0 = time.perf_counter()
    with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("fork")) as ex:
        res = list(ex.map(fn, range(n), [n] * n, [seconds] * n))
    wall = time.perf_counter() - t0
    done = sum(r[0] for r in res)
    units = sum(r[1] for r in res)
    what = "greedy tree verifications" if tree else "request verifications"
    return {"value": units / wall, "unit": UNIT, "cores": n, "kind": "oracle",
            "host_cores_visible": host,
            "worker_cap": f"{POOL_CAP} (the host's CPU share per GPU on the GPU boxes)",
            "sample": f"{done} oracle {what} on {n} forked workers (one per core, each cycling "
                      f"over its share of the {x.B} requests of the same seeded batch), fp64 "
                      f"numpy; wall time includes the pool start",
            "seconds": round(wall, 2)}


def graph_replay(calls, stream, replays, units, torch, launches_per_call=1):
    """One HIP graph holding every call of ``calls`` (bound to ``stream``) in order,
    replayed ``replays`` times; before timing, three replays are each checked
    against an eager run, with the outputs overwritten between replays.
    ``units`` counts the positions (or nodes) one call verifies."""
    import numpy as np

    s = stream
    with torch.cuda.stream(s):
        for c in calls:
            c.run()
    s.synchronize()
    ref = [[o.cpu().numpy() for o in c.out] for c in calls]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in calls:
            c.run()
    match = True
    for _ in range(3):
        with torch.cuda.stream(s):
            for c in calls:                 # eager work between replays: clobber the outputs
                for name, o in zip(c.out._fields, c.out):
                    if name != "status":    # the mask call ORs into its status word
                        o.fill_(-7)
            g.replay()
        s.synchronize()
        for c, r in zip(calls, ref):
            match &= all(np.array_equal(o.cpu().numpy(), e) for o, e in zip(c.out, r))
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        g.replay()
        ev0.record()
        for _ in range(replays):
            g.replay()
        ev1.record()
    s.synchronize()
    us_call = ev0.elapsed_time(ev1) * 1e3 / (replays * len(calls))
    return {"calls_per_graph": len(calls), "replays": replays, "us_per_call": us_call,
            "units_per_s": units / (us_call * 1e-6), "replays_match_eager": bool(match)}


def cpu_baseline_chain(x, seconds, gpu_out, space="prob"):
    """Oracle over the batch's requests in order (cycling) for about `seconds`."""
    import numpy as np

    import oracle
    t = x.widened(x.target)
    d = x.widened(x.draft)
    lens = x.lengths()
    done, pos, flagged, mismatch = 0, 0, 0, 0
    checked = set()
    t0 = time.perf_counter()
    while True:
        b = done % x.B
        k = int(lens[b])
        r = oracle.chain_verify_one(t[b, :k + 1], d[b, :k], x.tokens[b, :k], x.u_accept[b, :k],
                                    x.u_sample[b], x.lam, x.temperature, space)
        pos += k
        done += 1
        if b not in checked:
            checked.add(b)
            tok = np.full(x.K + 1, -1, dtype=np.int32)
            tok[:len(r.tokens)] = r.tokens
            same = gpu_out[0][b] == r.accepted and np.array_equal(gpu_out[1][b], tok)
            flagged += int(r.flagged)
            mismatch += int(not same and not r.flagged)
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    sample = (f"{done} oracle request verifications ({pos} drafted positions) cycling over the "
              f"{x.B} requests of the same seeded batch, fp64 numpy, one process")
    return ({"value": pos / el, "unit": UNIT, "cores": 1, "kind": "oracle", "sample": sample,
             "seconds": round(el, 2)},
            {"requests_checked": len(checked), "flagged": flagged, "unflagged_mismatches": mismatch})


def cpu_baseline_tree(x, seconds, gpu_out):
    import numpy as np

    import oracle
    t = x.widened(x.target)
    done, nodes, mismatch = 0, 0, 0
    checked = set()
    t0 = time.perf_counter()
    while True:
        b = done % x.B
        r = oracle.tree_greedy_one(t[b], x.parent[b], x.node_token[b])
        nodes += x.N
        done += 1
        if b not in checked:
            checked.add(b)
            tok = np.full(x.Dmax + 1, -1, dtype=np.int32)
            tok[:len(r.tokens)] = r.tokens
            mismatch += int(not (gpu_out[0][b] == r.accepted and np.array_equal(gpu_out[1][b], tok)))
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    sample = (f"{done} oracle greedy tree verifications ({nodes} nodes) cycling over the {x.B} "
              f"trees of the same seeded batch, fp64 numpy, one process")
    return ({"value": nodes / el, "unit": UNIT, "cores": 1, "kind": "oracle", "sample": sample,
             "seconds": round(el, 2)},
            {"requests_checked": len(checked), "unflagged_mismatches": mismatch})


def cpu_baseline_mask(x, seconds, gpu_mask, gpu_depth):
    import numpy as np

    import oracle
    done, nodes, mismatch = 0, 0, 0
    checked = set()
    W = gpu_mask.shape[2]
    t0 = time.perf_counter()
    while True:
        b = done % x.B
        r = oracle.tree_attention_mask_one(x.parent[b])
        nodes += x.N
        done += 1
        if b not in checked:
            checked.add(b)
            same = (np.array_equal(oracle.pack_mask_rows(r.mask, W), gpu_mask[b])
                    and np.array_equal(r.depth, gpu_depth[b]))
            mismatch += int(not same)
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    sample = (f"{done} oracle tree masks ({nodes} nodes) cycling over the {x.B} trees of the "
              f"same seeded batch, numpy, one process")
    return ({"value": nodes / el, "unit": "tree nodes masked/s", "cores": 1, "kind": "oracle",
             "sample": sample, "seconds": round(el, 2)},
            {"requests_checked": len(checked), "unflagged_mismatches": mismatch})


def bench_mask(args):
    """The tree-attention mask of the c5 trees: one mask call per step."""
    import numpy as np
    import torch

    from sampling_spec_verify_amd import specverify as sv
    from sampling_spec_verify_amd import synth

    sv.lib()
    x = synth.config("c5")
    par = torch.from_numpy(x.parent).to("cuda:0")
    call = sv.TreeMaskCall(par, x.N)
    W = call.out.mask.shape[2]
    graph = None
    if args.graph > 0:
        gs = torch.cuda.Stream()
        with torch.cuda.stream(gs):
            gcall = sv.TreeMaskCall(par, x.N, stream=gs)
        graph = graph_replay([gcall] * 64, gs, args.graph, x.B * x.N, torch)
    algo_bytes = 4 * (x.B * x.N + x.B * (x.N + 1) * W + x.B * (x.N + 1))
    for _ in range(args.warmup):
        call.run()
    torch.cuda.synchronize()
    K = args.steps
    every = args.time_every if args.time_every > 0 else 4
    timer = sv.KernelTimer(len(range(0, K, every)))
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(K):
        call.run(timer.pair(i // every) if i % every == 0 else None)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = np.array([timer.elapsed_ms(j) for j in range(len(timer.start))])
    timer.close()
    mask = call.out.mask.cpu().numpy().view(np.uint32)
    depth = call.out.depth.cpu().numpy()
    cpu, parity = (None, None)
    if args.cpu_seconds > 0:
        cpu, parity = cpu_baseline_mask(x, args.cpu_seconds, mask, depth)
    km = float(kern.mean())
    line = {
        "metric": "tree nodes masked/sec (tree-attention ancestor mask)",
        "value": x.B * x.N * K / wall, "unit": "tree nodes masked/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / K, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": f"c5mask: ancestor mask of the {synth.CONFIGS['c5']}",
                   "B": x.B, "N": x.N, "mask_words": W},
        "roofline": {"bound": "hbm", "achieved": algo_bytes / (km * 1e-3) / 1e9,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": algo_bytes / (km * 1e-3) / 1e9 / PEAK_HBM_GBS, "traffic": None,
                     "kernel": "tree_mask", "algorithmic_bytes_per_launch": algo_bytes,
                     "kernel_ms_mean": km, "kernel_ms_median": float(np.median(kern)),
                     "kernel_timing": f"HIP events attached to the launch in every {every}-th "
                                      f"timed step ({len(kern)} launches)",
                     "note": "launch-latency bound: a few KB per call"},
        "cpu_baseline": cpu, "gpu_ms_per_step": ev0.elapsed_time(ev1) / K,
        "graph_steady_state": graph,
        "status_word": int(call.out.status[0].item()), "parity_sample": parity,
    }
    print(json.dumps(line), flush=True)


def bench_alpha(args):
    """The acceptance-rate call on a chain workload: one call per step."""
    import numpy as np
    import torch

    import oracle
    from sampling_spec_verify_amd import specverify as sv
    from sampling_spec_verify_amd import synth

    sv.lib()
    x = synth.config(args.workload)
    elem = 2 if x.dtype == "bf16" else 4
    positions = x.positions()
    algo_bytes = 2 * 2 * x.V * elem * positions          # two passes over the drafted rows
    R = max(2, min(512, math.ceil(ROTATE_BYTES / (x.target.nbytes + x.draft.nbytes))))
    tgts = device_copies(x.target, x.dtype, R, torch)
    drfs = device_copies(x.draft, x.dtype, R, torch)
    dl = None if x.draft_len is None else torch.from_numpy(x.draft_len).to("cuda:0")
    calls = [sv.AcceptanceRateCall(tgts[i], drfs[i], x.lam, x.temperature, dl, space=args.space)
             for i in range(R)]
    for i in range(args.warmup):
        calls[i % R].run()
    torch.cuda.synchronize()
    K = args.steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(K):
        calls[i % R].run()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    alpha = calls[0].alpha.cpu().numpy()
    cpu = None
    if args.cpu_seconds > 0:
        t = x.widened(x.target)
        d = x.widened(x.draft)
        lens = x.lengths()
        done = pos = 0
        err = 0.0
        t1 = time.perf_counter()
        while time.perf_counter() - t1 < args.cpu_seconds:
            b = done % x.B
            k = int(lens[b])
            r = oracle.chain_verify_one(t[b, :k + 1], d[b, :k], x.tokens[b, :k],
                                        x.u_accept[b, :k], x.u_sample[b], x.lam, x.temperature,
                                        args.space)
            if done < x.B and k:
                err = max(err, float(np.abs(alpha[b, :k] - r.alpha).max()))
            pos += k
            done += 1
        el = time.perf_counter() - t1
        cpu = {"value": pos / el, "unit": "positions/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} oracle request verifications (each computes alpha), fp64 numpy",
               "seconds": round(el, 2), "alpha_max_abs_err": err}
    line = {
        "metric": "drafted positions/sec through the acceptance-rate call",
        "value": positions * K / wall, "unit": "positions/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / K, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{args.workload}: {synth.CONFIGS[args.workload]}",
                   "mixture_space": args.space, "buffer_sets_rotated": R},
        "step_hbm_gbps": algo_bytes * K / (wall * 1e9),
        "step_hbm_frac": algo_bytes * K / (wall * 1e9) / PEAK_HBM_GBS,
        "algorithmic_bytes_per_step": algo_bytes, "gpu_ms_per_step": ev0.elapsed_time(ev1) / K,
        "cpu_baseline": cpu, "status_word": int(calls[0].status[0].item()),
    }
    print(json.dumps(line), flush=True)


def bench_multi(args):
    """Multi-branch stochastic verification of the c5 trees: one call per step."""
    import numpy as np
    import torch

    import oracle
    from sampling_spec_verify_amd import specverify as sv
    from sampling_spec_verify_amd import synth

    sv.lib()
    x = synth.config("c5")
    dev = "cuda:0"
    R = max(2, min(512, math.ceil(ROTATE_BYTES / (x.target.nbytes + x.draft.nbytes))))
    tgts = device_copies(x.target, x.dtype, R, torch)
    drfs = device_copies(x.draft, x.dtype, R, torch)
    par = torch.from_numpy(x.parent).to(dev)
    tok = torch.from_numpy(x.node_token).to(dev)
    un = torch.from_numpy(x.u_node).to(dev)
    us = torch.from_numpy(x.u_sample).to(dev)
    ws = torch.empty(int(sv.lib().sv_tree_multi_workspace_bytes(x.B, x.N, x.V)),
                     dtype=torch.uint8, device=dev)

    def call(i):
        return sv.tree_verify_multi(tgts[i % R], drfs[i % R], par, tok, un, us, x.Dmax, x.lam,
                                    x.temperature, args.space, workspace=ws)
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    K = args.steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(K):
        out = call(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    g = [o.cpu().numpy() for o in out]
    cpu, parity = None, None
    if args.cpu_seconds > 0:
        t, d = x.widened(x.target), x.widened(x.draft)
        done = nodes = mism = flagged = 0
        t1 = time.perf_counter()
        while time.perf_counter() - t1 < args.cpu_seconds:
            b = done % x.B
            r = oracle.tree_multi_one(t[b], d[b], x.parent[b], x.node_token[b], x.u_node[b],
                                      x.u_sample[b], x.lam, x.temperature, args.space, x.Dmax)
            if done < x.B:
                ref = np.full(x.Dmax + 1, -1, dtype=np.int32)
                ref[:len(r.tokens)] = r.tokens
                same = g[0][b] == r.accepted and np.array_equal(g[1][b], ref)
                flagged += int(r.flagged)
                mism += int(not same and not r.flagged)
            nodes += x.N
            done += 1
        el = time.perf_counter() - t1
        cpu = {"value": nodes / el, "unit": "tree nodes/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} oracle multi-branch tree walks cycling over the {x.B} trees, "
                         f"fp64 numpy, one process", "seconds": round(el, 2)}
        parity = {"requests_checked": min(done, x.B), "flagged": flagged,
                  "unflagged_mismatches": mism}
    line = {
        "metric": "draft-tree nodes/sec through multi-branch stochastic verification",
        "value": x.B * x.N * K / wall, "unit": "tree nodes/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / K, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"c5multi: {synth.CONFIGS['c5']}, per-node uniforms",
                   "mixture_space": args.space, "lambda": x.lam, "buffer_sets_rotated": R},
        "gpu_ms_per_step": ev0.elapsed_time(ev1) / K, "cpu_baseline": cpu,
        "parity_sample": parity, "status_word": int(g[4][0]),
        "accepted_depths": g[0].tolist(),
        "note": "a row-statistics launch over the tree rows, then up to 32 cooperating "
                "512-thread blocks walk each tree; bound by the chain of barriers between "
                "the walk's vocabulary passes",
    }
    print(json.dumps(line), flush=True)


def bench_path(args):
    """Path mode on the c5 trees: chain acceptance along each tree's seeded root-to-leaf
    path (target rows [0, n_1..n_d], draft rows [0, n_1..n_{d-1}]); one call per step."""
    import numpy as np
    import torch

    import oracle
    from sampling_spec_verify_amd import specverify as sv
    from sampling_spec_verify_amd import synth

    sv.lib()
    x = synth.config("c5")
    dev = "cuda:0"
    elem = 2 if x.dtype == "bf16" else 4
    # drafted positions of each path: its node ids up to the -1 terminator
    dlen = np.array([int(np.argmax(np.append(p, -1) < 1)) for p in x.path])
    positions = int(dlen.sum())
    algo_bytes = 2 * x.V * elem * positions          # the row-statistics stream
    R = max(2, min(512, math.ceil(ROTATE_BYTES / (x.target.nbytes + x.draft.nbytes))))
    tgts = device_copies(x.target, x.dtype, R, torch)
    drfs = device_copies(x.draft, x.dtype, R, torch)
    tok = torch.from_numpy(x.node_token).to(dev)
    path = torch.from_numpy(x.path).to(dev)
    ua = torch.from_numpy(x.u_accept).to(dev)
    us = torch.from_numpy(x.u_sample).to(dev)
    calls = [sv.TreePathCall(tgts[i], drfs[i], tok, path, ua, us, x.lam, x.temperature,
                             space=args.space) for i in range(R)]
    for i in range(args.warmup):
        calls[i % R].run()
    torch.cuda.synchronize()
    K = args.steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(K):
        calls[i % R].run()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    g = [o.cpu().numpy() for o in calls[0].out]
    graph = None
    if args.graph > 0:
        gs = torch.cuda.Stream()
        with torch.cuda.stream(gs):
            gcalls = [sv.TreePathCall(tgts[i], drfs[i], tok, path, ua, us, x.lam, x.temperature,
                                      stream=gs, space=args.space) for i in range(R)]
        graph = graph_replay(gcalls, gs, args.graph, positions, torch)
    cpu, parity = None, None
    if args.cpu_seconds > 0:
        t, d = x.widened(x.target), x.widened(x.draft)
        done = pos = mism = flagged = 0
        t1 = time.perf_counter()
        while time.perf_counter() - t1 < args.cpu_seconds:
            b = done % x.B
            r = oracle.tree_path_one(t[b], d[b], x.node_token[b], x.path[b], x.u_accept[b],
                                     x.u_sample[b], x.lam, x.temperature, args.space)
            if done < x.B:
                ref = np.full(x.path.shape[1] + 1, -1, dtype=np.int32)
                ref[:len(r.tokens)] = r.tokens
                same = g[0][b] == r.accepted and np.array_equal(g[1][b], ref)
                flagged += int(r.flagged)
                mism += int(not same and not r.flagged)
            pos += int(dlen[b])
            done += 1
        el = time.perf_counter() - t1
        cpu = {"value": pos / el, "unit": UNIT, "cores": 1, "kind": "oracle",
               "sample": f"{done} oracle path verifications ({pos} drafted positions) cycling "
                         f"over the {x.B} trees, fp64 numpy, one process",
               "seconds": round(el, 2)}
        parity = {"requests_checked": min(done, x.B), "flagged": flagged,
                  "unflagged_mismatches": mism}
    line = {
        "metric": "verified path positions/sec through path-mode tree verification",
        "value": positions * K / wall, "unit": UNIT, "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / K, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"c5path: {synth.CONFIGS['c5']}, seeded root-to-leaf paths",
                   "path_lengths": dlen.tolist(), "mixture_space": args.space,
                   "lambda": x.lam, "temperature": x.temperature, "buffer_sets_rotated": R},
        "step_hbm_gbps": algo_bytes * K / (wall * 1e9),
        "step_hbm_frac": algo_bytes * K / (wall * 1e9) / PEAK_HBM_GBS,
        "algorithmic_bytes_per_step": algo_bytes, "gpu_ms_per_step": ev0.elapsed_time(ev1) / K,
        "graph_steady_state": graph, "cpu_baseline": cpu, "parity_sample": parity,
        "status_word": int(g[3][0]),
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the verify step is data-parallel over requests and "
              f"this build runs on a single MI355X; --gpus {args.gpus} is not supported.",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.workload == "c5mask":
        bench_mask(args)
        return
    if args.workload == "c5multi":
        bench_multi(args)
        return
    if args.workload == "c5path":
        bench_path(args)
        return
    if args.alpha:
        bench_alpha(args)
        return

    from sampling_spec_verify_amd import synth

    x = synth.config(args.workload)
    tree = args.workload == "c5"
    cpu_pool = None
    if args.cpu_seconds > 0 and args.cpu_pool_seconds > 0:
        cpu_pool = cpu_pool_baseline(x, tree, args.cpu_pool_seconds, args.space)

    import numpy as np
    import torch

    from sampling_spec_verify_amd import specverify as sv

    sv.lib()
    elem = 2 if x.dtype == "bf16" else 4
    if tree:
        positions = x.B * x.N
        algo_bytes = x.B * (x.N + 1) * x.V * elem
        footprint = x.target.nbytes
    else:
        positions = x.positions()
        algo_bytes = 2 * x.V * elem * positions
        footprint = x.target.nbytes + x.draft.nbytes
    R = max(2, min(512, math.ceil(ROTATE_BYTES / footprint)))

    dev = "cuda:0"
    tgts = device_copies(x.target, x.dtype, R, torch)
    if tree:
        par = torch.from_numpy(x.parent).to(dev)
        ntok = torch.from_numpy(x.node_token).to(dev)
        calls = [sv.TreeGreedyCall(tgts[i], par, ntok, x.Dmax) for i in range(R)]

        def step(i, events=None):
            calls[i % R].run(events)
    else:
        drfs = device_copies(x.draft, x.dtype, R, torch)
        tok = torch.from_numpy(x.tokens).to(dev)
        ua = torch.from_numpy(x.u_accept).to(dev)
        us = torch.from_numpy(x.u_sample).to(dev)
        dl = None if x.draft_len is None else torch.from_numpy(x.draft_len).to(dev)
        calls = [sv.ChainCall(tgts[i], drfs[i], tok, ua, us, x.lam, x.temperature, dl,
                              space=args.space) for i in range(R)]

        def step(i, events=None):
            c = calls[i % R]
            if events is None:
                c.run()
            else:
                c.row_stats(events)
                c.accept_resample()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    every = args.time_every
    timed = list(range(0, K, every)) if every > 0 else []
    timer = sv.KernelTimer(len(timed)) if timed else None
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(K):
        step(i, timer.pair(i // every) if timed and i % every == 0 else None)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    gpu_ms = ev0.elapsed_time(ev1)
    in_loop_ms = np.array([timer.elapsed_ms(j) for j in range(len(timed))]) if timed else None
    if timer:
        timer.close()
    ms_per_step = wall * 1e3 / K
    value = positions * K / wall
    # the greedy call's one launch covers trees of at most 64 nodes, 1024 trees
    fold = tree and x.N + 1 <= 64 and x.B <= 1024
    kname = ("greedy_fold" if fold else "row_argmax") if tree else "row_stats"
    traffic = load_traffic(kname, args.workload)

    out = calls[0].out
    torch.cuda.synchronize()
    status = int(out.status[0].item())
    gpu_out = [o.cpu().numpy() for o in out]

    # the dominant kernel (and the chain's accept / resample kernel) over
    # launch-attached events, in a leg of its own: one full call per rep through
    # the two stage calls, buffer sets rotated as in the timed steps
    reps = max(1, args.kernel_reps)
    kt = sv.KernelTimer(reps)
    mt = None if tree else sv.KernelTimer(reps)
    for i in range(reps):
        c = calls[i % R]
        if tree:
            c.run(kt.pair(i))
        else:
            c.row_stats(kt.pair(i))
            c.accept_resample(mt.pair(i))
    torch.cuda.synchronize()
    first_ms = np.array([kt.elapsed_ms(i) for i in range(reps)])
    kt.close()
    kern_ms = float(np.median(first_ms))
    achieved = algo_bytes / (kern_ms * 1e-3) / 1e9
    mass = None
    if mt is not None:
        mass_ms = np.array([mt.elapsed_ms(i) for i in range(reps)])
        mt.close()
        lens = x.lengths()
        # the sampling row(s) each request reads: target and draft row at a
        # rejection, the target's bonus row when every draft is accepted
        mass_bytes = int(sum((2 if gpu_out[0][b] < lens[b] else 1) * x.V * elem
                             for b in range(x.B)))
        mm = float(np.median(mass_ms))
        mass = {"kernel": "resolve_mass", "bound": "hbm",
                "algorithmic_bytes_per_launch": mass_bytes,
                "rejected_requests": int(sum(gpu_out[0][b] < lens[b] for b in range(x.B))),
                "kernel_ms_median": mm, "kernel_ms_p10": float(np.percentile(mass_ms, 10)),
                "kernel_ms_p90": float(np.percentile(mass_ms, 90)),
                "achieved": mass_bytes / (mm * 1e-3) / 1e9,
                "frac": mass_bytes / (mm * 1e-3) / 1e9 / PEAK_HBM_GBS}
    argmax_only = None
    if fold:
        at = sv.KernelTimer(reps)
        for i in range(reps):
            c = calls[i % R]
            c.row_argmax(at.pair(i))
            c.walk()
        torch.cuda.synchronize()
        am_ms = np.array([at.elapsed_ms(i) for i in range(reps)])
        at.close()
        amm = float(np.median(am_ms))
        argmax_only = {"kernel": "row_argmax", "note": "the two-launch form's first kernel: the same "
                       "row stream and chunk argmax, without the walks",
                       "kernel_ms_median": amm, "kernel_ms_p10": float(np.percentile(am_ms, 10)),
                       "kernel_ms_p90": float(np.percentile(am_ms, 90)),
                       "achieved": algo_bytes / (amm * 1e-3) / 1e9,
                       "frac": algo_bytes / (amm * 1e-3) / 1e9 / PEAK_HBM_GBS}
    graph = None
    if args.graph > 0:
        gs = torch.cuda.Stream()
        with torch.cuda.stream(gs):
            if tree:
                gcalls = [sv.TreeGreedyCall(tgts[i], par, ntok, x.Dmax, stream=gs) for i in range(R)]
            else:
                gcalls = [sv.ChainCall(tgts[i], drfs[i], tok, ua, us, x.lam, x.temperature, dl,
                                       stream=gs, space=args.space) for i in range(R)]
        graph = graph_replay(gcalls, gs, args.graph, positions, torch)
    ceiling = None
    if not args.no_stream_ceiling:
        ceiling = read_stream_ceiling(algo_bytes, torch, sv)

    cpu = None
    parity = None
    if args.cpu_seconds > 0:
        if tree:
            cpu, parity = cpu_baseline_tree(x, args.cpu_seconds, gpu_out)
        else:
            cpu, parity = cpu_baseline_chain(x, args.cpu_seconds, gpu_out, args.space)

    config = {"workload": f"{args.workload}: {synth.CONFIGS[args.workload]}",
              "B": x.B, "V": x.V, "logits": x.dtype,
              "positions_per_step": positions, "buffer_sets_rotated": R}
    if not tree:
        config.update({"K": x.K, "ragged": x.draft_len is not None, "lambda": x.lam,
                       "temperature": x.temperature, "mixture_space": args.space})
    line = {
        "metric": METRIC,
        "value": value,
        "unit": UNIT,
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": kname, "algorithmic_bytes_per_launch": algo_bytes,
                     "kernel_ms_median": kern_ms, "kernel_ms_mean": float(first_ms.mean()),
                     "kernel_ms_p10": float(np.percentile(first_ms, 10)),
                     "kernel_ms_p90": float(np.percentile(first_ms, 90)),
                     "kernel_timing": f"median of {reps} launch-attached HIP event pairs, one per "
                                      f"full call in a leg after the timed steps",
                     "in_loop_kernel_ms_median": (float(np.median(in_loop_ms))
                                                  if in_loop_ms is not None else None),
                     "read_stream": ceiling,
                     "frac_of_read_stream": (achieved / ceiling["gbs_median"]) if ceiling else None},
        "mass_kernel": mass,
        "argmax_only": argmax_only,
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_pool,
        "graph_steady_state": graph,
        "step_hbm_gbps": algo_bytes * K / (wall * 1e9),
        "step_hbm_frac": algo_bytes * K / (wall * 1e9) / PEAK_HBM_GBS,
        "gpu_ms_per_step": gpu_ms / K,
        "status_word": status,
        "parity_sample": parity,
        "kernel_source_hash": kernel_source_hash(kname),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
