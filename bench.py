#!/usr/bin/env python3
"""Decode query-rows/s and indexer-scan HBM bandwidth of the CSA2 sparse decode path on
one MI355X.

One step = one csa2_decode launch chain over one batch: indexer scan of every entry, coarse
block filter, fine top-512, and joint-softmax attention over the selected FP4 entries
plus the FP8 window.  The default workload is the 128K-context decode (1 request x 1
row, 131072 tokens pooled to 65536 entries).  Inputs are synthetic (seeded) and sit in
HBM before timing starts; the steps rotate over enough device copies of the inputs
that no step finds its data in the 256 MB last-level cache, so every step reads HBM.

The timed steps are replays of a HIP graph that holds one captured decode step per
input copy (the eager per-call time is reported beside it).  Per-stage kernel times
come from HIP events that csa2_decode records between its kernels on the launch
stream, captured into the same graph, inside the timed region.  A second timed loop runs the
scan kernel alone on a 64 x 128K batch (285 MB of keys, larger than the cache) for the
bandwidth-at-scale figure.  The oracle (fp64, CPU) is timed on a bounded sample.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0        # dense bf16 MFMA
MALL_BYTES = 256 << 20           # last-level (Infinity) cache


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


def make_events(hip, n):
    arr = (ctypes.c_void_p * n)()
    for i in range(n):
        h = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        arr[i] = h
    return arr


def elapsed_ms(hip, a, b) -> float:
    f = ctypes.c_float()
    rc = hip.hipEventElapsedTime(ctypes.byref(f), a, b)
    if rc != 0:
        raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
    return float(f.value)


def replicate(dw, n):
    """n device copies of a workload's cache pools and queries (same descriptor)."""
    import torch
    from synth.device import DeviceWorkload
    reps = [dw]
    for _ in range(n - 1):
        reps.append(DeviceWorkload(rg=dw.rg, idx_k=dw.idx_k.clone(), main_kv=dw.main_kv.clone(),
                                   blk_sum=dw.blk_sum.clone(), swa=dw.swa.clone(), swa_scale=dw.swa_scale.clone(),
                                   q=dw.q.clone(), q_idx=dw.q_idx.clone(), w=dw.w.clone()))
    torch.cuda.synchronize()
    return reps


def graph_time_ms(hip, fns, replays: int, warm: int = 2) -> float:
    """Capture fns (each enqueues one launch chain) into one HIP graph, replay it, and
    return the mean time per fn call from events recorded on the stream around the
    replays."""
    import torch
    from sparse_decode_attention_csa2_amd import capture_calls
    g = capture_calls(fns)
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    ev = make_events(hip, 2)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    hip.hipEventRecord(ev[0], st)
    for _ in range(replays):
        g.replay()
    hip.hipEventRecord(ev[1], st)
    torch.cuda.synchronize()
    return elapsed_ms(hip, ev[0], ev[1]) / (replays * len(fns))


def touched_bytes(wl) -> int:
    """Bytes a decode step reads from the pools (for sizing the replica rotation)."""
    R = wl.num_rows
    return (wl.total_entries * 68 + int(wl.block_off[-1]) * 256 + R * (512 * 288 + 128 * 516 + 64 * 512 * 2))


def algorithmic(wl):
    """Algorithmic bytes / flops per launch of each stage."""
    R = wl.num_rows
    nb = int(wl.block_off[-1])
    scan = wl.total_entries * 68 + nb * 256 + R * (8 * 128 * 2 + 8 * 4)
    attn_bytes = R * (512 * 288 + 128 * (512 + 4) + 64 * 512 * 2 + 64 * 512 * 4 + 64 * 4)
    attn_flops = R * 4 * 64 * (512 + 128) * 512
    return scan, attn_bytes, attn_flops


def cpu_baseline(wl, seconds: float):
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = min(16, len(os.sched_getaffinity(0)))
    with threadpool_limits(limits=cores):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        t0 = time.perf_counter()
        rows = 0
        while True:
            oracle.decode(wl)
            rows += wl.num_rows
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "query-rows/s", "cores": int(used), "kind": "oracle",
            "sample": f"{wl.name}: the whole path in fp64 for all {wl.num_rows} row(s) "
                      f"({wl.total_entries} entries scanned per pass), repeated {rows // wl.num_rows}x "
                      f"over {dt:.1f}s"}


def scan_at_scale(csa2, hip, steps: int):
    """Scan kernel alone on 64 x 128K requests (285 MB of keys per launch)."""
    import torch
    from synth import make_workload
    from synth.device import upload
    wl = make_workload("long_128k_x64", 1, [65536] * 64, rows_per_req=1, n_needles=16, scan_only=True)
    dw = upload(wl)
    scores = torch.empty((wl.num_rows, wl.max_entries), dtype=torch.float32, device="cuda")
    idx2 = dw.idx_k.clone()          # two copies (570 MB) alternate: no launch finds its keys cached
    fns = [lambda k=k: csa2.index_score(dw.rg, k, dw.q_idx, dw.w, scores=scores) for k in (dw.idx_k, idx2)]
    for f in fns:
        f()
    ms = graph_time_ms(hip, fns, replays=max(5, steps // 2))
    algo = wl.total_entries * 68 + wl.num_rows * (8 * 128 * 2 + 8 * 4)
    gbs = algo / (ms * 1e-3) / 1e9
    return {"workload": "64 requests x 131072 tokens (65536 entries each), scan kernel alone, graph-launched",
            "bytes_per_launch": algo, "us_per_launch": ms * 1e3, "achieved_GBs": gbs,
            "frac_of_peak": gbs / HBM_PEAK_GBS}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=1, help="workload id (default 1: 128K-context decode)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-scale", action="store_true", help="skip the 64 x 128K scan-bandwidth loop")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import sparse_decode_attention_csa2_amd as csa2
    from synth import make_config
    from synth.device import upload

    if not os.path.exists(csa2.LIB_PATH):
        from __graft_entry__ import build
        build()
    torch.cuda.set_device(0)
    hip = _hip()
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    wl = make_config(args.config)
    dw = upload(wl)
    n_rep = max(2, math.ceil(2 * MALL_BYTES / max(1, touched_bytes(wl))) + 1)
    reps = replicate(dw, n_rep)
    decs = [csa2.Decoder(*r.decode_inputs(), k=wl.k, n_keep=wl.n_keep, sm_scale=wl.sm_scale,
                         keep_intermediates=False) for r in reps]
    for d in decs:
        d.run()
    torch.cuda.synchronize()
    K, W = args.steps, args.warmup
    E = csa2.DECODE_EVENTS
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    outer = make_events(hip, 2)

    # Eager launches (reference): one csa2_decode call per step from Python.
    for i in range(W):
        decs[i % n_rep].run()
    torch.cuda.synchronize()
    hip.hipEventRecord(outer[0], st)
    n_eager = min(K, 4 * n_rep)
    for i in range(n_eager):
        decs[i % n_rep].run()
    hip.hipEventRecord(outer[1], st)
    torch.cuda.synchronize()
    eager_ms = elapsed_ms(hip, outer[0], outer[1]) / n_eager

    # Eager per-stage breakdown (events between the kernels; includes dispatch gaps).
    evs = [make_events(hip, E) for _ in range(n_rep)]
    for i in range(n_rep):
        decs[i].run(events=evs[i])
    torch.cuda.synchronize()
    stage_names = ["scan", "select", "attention", "merge"]
    stage_ms = {n: float(np.mean([elapsed_ms(hip, evs[i][j], evs[i][j + 1]) for i in range(n_rep)]))
                for j, n in enumerate(stage_names)}

    # Timed region: replays of a HIP graph holding one decode step per input replica.
    graph = csa2.capture_graph(decs)
    reps_needed = max(1, math.ceil(K / n_rep))
    for _ in range(max(1, math.ceil(W / n_rep))):
        graph.replay()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    hip.hipEventRecord(outer[0], st)
    for _ in range(reps_needed):
        graph.replay()
    hip.hipEventRecord(outer[1], st)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    K = reps_needed * n_rep
    total_ms = elapsed_ms(hip, outer[0], outer[1])
    ms_step = total_ms / K

    # Kernel timing for the rooflines: each kernel alone, launched back to back from a
    # graph over the same cold input copies, events on the launch stream around it.
    scan_out = torch.empty((wl.num_rows, max(1, wl.max_entries)), dtype=torch.float32, device="cuda")
    scan_fns = [lambda r=r: csa2.index_score(r.rg, r.idx_k, r.q_idx, r.w, scores=scan_out) for r in reps]
    scan_ms = graph_time_ms(hip, scan_fns, replays=max(3, reps_needed))
    d0 = csa2.Decoder(*reps[0].decode_inputs(), k=wl.k, n_keep=wl.n_keep, sm_scale=wl.sm_scale)
    d0.run()
    torch.cuda.synchronize()
    attn_out = torch.empty((wl.num_rows, 64, 512), dtype=torch.float32, device="cuda")
    attn_lse = torch.empty((wl.num_rows, 64), dtype=torch.float32, device="cuda")
    attn_ws = torch.empty((max(256, csa2.sparse_attn_workspace_size(reps[0].rg, wl.k)),), dtype=torch.uint8,
                          device="cuda")
    attn_fns = [lambda r=r: csa2.sparse_attn(r.rg, r.q, r.main_kv, d0.sel_idx, d0.n_sel, r.swa, r.swa_scale,
                                             wl.sm_scale, out=attn_out, lse=attn_lse, ws=attn_ws) for r in reps]
    attn_ms = graph_time_ms(hip, attn_fns, replays=max(3, reps_needed))

    scan_b, attn_b, attn_f = algorithmic(wl)
    scan_b_entries = wl.total_entries * 68 + wl.num_rows * (8 * 128 * 2 + 8 * 4)
    scan_gbs = scan_b_entries / (scan_ms * 1e-3) / 1e9
    attn_gbs = attn_b / (attn_ms * 1e-3) / 1e9
    attn_tfs = attn_f / (attn_ms * 1e-3) / 1e12
    rl_scan = {"kernel": "indexer scan (csa2_index_score, every entry)", "bound": "hbm", "achieved": scan_gbs,
               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": scan_gbs / HBM_PEAK_GBS, "traffic": None,
               "bytes_per_launch": scan_b_entries, "us_per_launch": scan_ms * 1e3}
    rl_attn = {"kernel": "sparse attention (csa2_sparse_attn: attention + merge kernels)", "bound": "hbm",
               "achieved": attn_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": attn_gbs / HBM_PEAK_GBS,
               "traffic": None, "bytes_per_launch": attn_b, "us_per_launch": attn_ms * 1e3,
               "mfma_TFLOPs": attn_tfs, "mfma_frac": attn_tfs / BF16_PEAK_TFLOPS}

    res = {
        "metric": "decode query-rows/s + indexer-scan HBM GB/s (% of peak) at 128K ctx, top-512",
        "value": wl.num_rows * K / (total_ms * 1e-3),
        "unit": "query-rows/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4/fp8 in, bf16 mfma, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.num_requests} request(s) x {wl.num_rows // max(1, wl.num_requests)} "
                               f"row(s), {wl.total_entries} entries, top-{wl.k}, keep {wl.n_keep}+newest blocks, "
                               f"128-token FP8 window",
                   "requests": wl.num_requests, "rows": wl.num_rows, "entries": wl.total_entries,
                   "input_replicas": n_rep},
        "roofline": rl_scan,
        "attention_roofline": rl_attn,
        "launch": "hip graph replay (one captured decode step per input replica)",
        "eager_ms_per_step": eager_ms,
        "stages_us_eager": {k: v * 1e3 for k, v in stage_ms.items()},
        "wall_s_timed": t_wall,
    }
    if not args.no_scale:
        res["scan_at_scale"] = scan_at_scale(csa2, hip, steps=max(20, min(200, K // 10)))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
