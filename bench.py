#!/usr/bin/env python3
"""Decode query-rows/s and indexer-scan HBM bandwidth of the CSA2 sparse decode path on
one MI355X.

One step = one csa2_decode launch chain over one batch: indexer scan of every entry, coarse
block filter, fine top-512, and joint-softmax attention over the selected FP4 entries
plus the FP8 window.  The headline workload is the 128K-context decode (1 request x 1
row, 131072 tokens pooled to 65536 entries).  Inputs are synthetic (seeded) and sit in
HBM before timing starts; the steps rotate over enough device copies of the inputs
that no step finds its data in the 256 MB last-level cache, so every step reads HBM.

The timed region is exactly --steps decode steps: csa2_decode calls rotating over the
input copies, enqueued behind a spin kernel so that the GPU runs them back to back;
steady-state figures over at least 2,000 steps (the same calls, and replays of a HIP
graph holding one step per input copy) and an eager per-stage split are reported beside
it.  The other workloads (tiny, batched, verify,
1M-unpooled, 64 x 128K, paged pools, the MXFP8 route, the candidate-only scan) are timed
the same way and reported per workload.  The roofline entry is the indexer scan on the
64 x 128K batch (285 MB of FP4 keys per launch, launched alone over two alternating
input copies), timed over runs of 200 back-to-back launches between a HIP event pair on
the launch stream (a 20-launch burst is reported beside it); its HBM traffic comes from
the committed counter summary when that summary was taken on the current scan sources.
The oracle (fp64, CPU) is timed on a bounded sample: all cores, one thread, and its scan
alone.

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
    lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
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


def cache_write_timing(csa2, hip) -> dict:
    """csa2_cache_write (pooling, RMSNorm, FP4 quantisation, record and summary writes)
    for the verify batch (8 requests x 6 rows) and for 64 requests x 2 rows: back-to-back
    calls behind a spin kernel (one call is too short for a graph replay per call to
    measure anything but the replay's own launch cost)."""
    import torch
    from synth import make_config, make_write_inputs
    from synth.device import upload
    out = {}
    for name, wl in (("verify_8x6", make_config(3)), ("decode_64x2", None)):
        if wl is None:
            from synth import make_workload
            wl = make_workload("decode_64x2", 7, [4096] * 64, rows_per_req=2, n_needles=0)
        w = make_write_inputs(wl, 70)
        dw = upload(wl)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16
                                         else np.ascontiguousarray(a)).cuda()
        args = (dw.rg, dev(w["row_pos"]), dev(w["kv_tok"]), dev(w["idx_tok"]), dev(w["ring_kv"]), dev(w["ring_idx"]),
                dev(w["gamma_kv"]), dev(w["gamma_idx"]), dw.main_kv, dw.idx_k, dw.blk_sum)
        csa2.cache_write(*args)
        torch.cuda.synchronize()
        ms = graph_kernel_ms(hip, [lambda: csa2.cache_write(*args)], launches=200)
        entries = int(sum(1 for p in w["row_pos"] if p % 2 == 1))
        out[name] = {"rows": wl.num_rows, "entries_written": entries, "us_per_call": ms * 1e3}
        del dw, args
        torch.cuda.empty_cache()
    return out


def touched_bytes(wl) -> int:
    """Bytes a decode step reads from the pools (for sizing the replica rotation)."""
    R = wl.num_rows
    return (wl.total_entries * 68 + int(wl.block_off[-1]) * 256 + R * (512 * 288 + 128 * 516 + 64 * 512 * 2))


def step_bytes(wl) -> int:
    """Algorithmic bytes of one decode step: every request's indexer keys (68 B per entry)
    and block summaries (256 B per 64-entry block), each row's indexer query and weights,
    and per row the attention's 512 selected records, 128 window tokens, query and
    outputs.  The select's reads (at most 4,160 scores per row) are left out."""
    nb = sum((wl.n_entries(b) + 63) // 64 for b in range(wl.num_requests))
    ne = sum(wl.n_entries(b) for b in range(wl.num_requests))
    return ne * 68 + nb * 256 + wl.num_rows * (8 * 128 * 2 + 8 * 4) + attn_bytes(wl)


def cpu_baseline(wl, seconds: float):
    """The oracle (fp64 numpy, as it stands) on the headline workload, on this host: the
    whole path on every available core (BLAS pool = the process's CPU affinity), the
    same on one thread, and its indexer scan alone (effective GB/s over the 68-B keys)."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    avail = len(os.sched_getaffinity(0))

    def rows_per_s(threads, budget):
        with threadpool_limits(limits=threads):
            used = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
            t0 = time.perf_counter()
            rows = 0
            while True:
                oracle.decode(wl)
                rows += wl.num_rows
                if time.perf_counter() - t0 >= budget:
                    break
            return rows / (time.perf_counter() - t0), int(used), rows // wl.num_rows

    all_rate, used, passes = rows_per_s(avail, seconds)
    one_rate, _, one_passes = rows_per_s(1, seconds / 2)
    with threadpool_limits(limits=avail):
        t0 = time.perf_counter()
        n_scan = 0
        while True:
            for b in range(wl.num_requests):
                oracle.request_scores(wl, b)
            n_scan += 1
            if time.perf_counter() - t0 >= seconds / 4:
                break
        scan_s = (time.perf_counter() - t0) / n_scan
    scan_bytes_all = wl.total_entries * 68
    return {"value": all_rate, "unit": "query-rows/s", "cores": used, "kind": "oracle",
            "host_cores_available": avail, "host_cpu_count": os.cpu_count(), "threads_used": used,
            "value_1_thread": one_rate,
            "scan_GBs": scan_bytes_all / scan_s / 1e9,
            "sample": f"{wl.name}: the whole path in fp64 for all {wl.num_rows} row(s) "
                      f"({wl.total_entries} entries scanned per pass), {passes} passes over {seconds:.0f} s on "
                      f"{used} BLAS threads ({avail} cores available), {one_passes} passes on 1 thread; "
                      f"scan_GBs: the oracle's indexer scores alone over the {scan_bytes_all} key bytes"}


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "sparse_decode_attention_csa2_amd", "csrc")


def sources_digest(names) -> str:
    """sha256 over the named kernel sources (ties a counter summary to the code it measured)."""
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


SCAN_SOURCES = ("scan.hip", "csa2_dev.h", "csa2_internal.h")
ATTN_SOURCES = ("attn.hip", "csa2_dev.h", "csa2_internal.h")


def read_counter_summary(name: str) -> dict:
    """key: value lines of a committed counter summary (empty if absent)."""
    path = os.path.join(PROFILES, name)
    out = {}
    if not os.path.exists(path):
        return out
    with open(path) as f:
        for line in f:
            line = line.strip().lstrip("-* ").strip("`")
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                out[k.strip()] = v.strip().strip("`")
    return out


def graph_kernel_ms(hip, fns, launches: int, repeats: int = 5) -> float:
    """Average duration of one launch chain of fns, from a HIP event pair on the launch
    stream around `launches` back-to-back launches (cycling over fns); the median over
    `repeats` such runs.  The stream is held by a spin kernel while the launches are
    enqueued, so the GPU runs them back to back and the events do not include host
    submission time."""
    import torch
    n = max(1, launches)
    for f in fns[:4]:
        f()
    torch.cuda.synchronize()
    ev = make_events(hip, 2)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    runs = []
    for _ in range(repeats):
        torch.cuda._sleep(int(2.0e9 * (n * 60e-6 + 2e-3)))
        hip.hipEventRecord(ev[0], st)
        for i in range(n):
            fns[i % len(fns)]()
        hip.hipEventRecord(ev[1], st)
        torch.cuda.synchronize()
        runs.append(elapsed_ms(hip, ev[0], ev[1]) / n)
    return float(np.median(runs))


def measure_decode(csa2, hip, wl, steps: int, warmup: int, max_reps: int = 128, qp_route: int = 0,
                   scan_mode: int = 0):
    """Decode steps over rotating input copies; returns timings.

    The timed region is exactly ``steps`` decode steps: csa2_decode calls rotating over
    the input copies, enqueued behind a spin kernel and bracketed by a HIP event pair on
    the launch stream (synchronised on both sides).  Beside it: an eager per-stage split,
    per-step latency percentiles and two steady-state figures over at least 2,000 steps
    (the same eager calls, and replays of one HIP graph holding a step per input copy)."""
    import torch
    from synth.device import upload
    dw = upload(wl)
    n_rep = min(max_reps, max(2, math.ceil(2 * MALL_BYTES / max(1, touched_bytes(wl))) + 1))
    reps = replicate(dw, n_rep)
    decs = [csa2.Decoder(*r.decode_inputs(), k=wl.k, n_keep=wl.n_keep, sm_scale=wl.sm_scale,
                         keep_intermediates=False, qp_route=qp_route, scan_mode=scan_mode) for r in reps]
    for d in decs:
        d.run()
    torch.cuda.synchronize()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    outer = make_events(hip, 2)
    # Eager per-stage split (events between the kernels; includes dispatch gaps).
    E = csa2.DECODE_EVENTS
    evs = [make_events(hip, E) for _ in range(n_rep)]
    for i in range(n_rep):
        decs[i].run(events=evs[i])
    torch.cuda.synchronize()
    names = ["scan", "select", "attention", "merge"]
    stages = {n: float(np.mean([elapsed_ms(hip, evs[i][j], evs[i][j + 1]) for i in range(n_rep)])) * 1e3
              for j, n in enumerate(names)}
    # Per-step latency distribution: one event pair around each decode step, the steps
    # enqueued behind a spin kernel so they run back to back.
    n_lat = min(200, max(20, 2 * n_rep))
    lev = make_events(hip, 2 * n_lat)
    torch.cuda._sleep(int(2.0e9 * (n_lat * 80e-6 + 2e-3)))
    for i in range(n_lat):
        hip.hipEventRecord(lev[2 * i], st)
        decs[i % n_rep].run()
        hip.hipEventRecord(lev[2 * i + 1], st)
    torch.cuda.synchronize()
    lat = np.array([elapsed_ms(hip, lev[2 * i], lev[2 * i + 1]) for i in range(n_lat)]) * 1e3
    lat_us = {"p10": float(np.percentile(lat, 10)), "p50": float(np.percentile(lat, 50)),
              "p90": float(np.percentile(lat, 90)), "steps": n_lat}
    # Timed region: exactly `steps` csa2_decode calls, rotating over the input copies,
    # enqueued behind a spin kernel (the GPU runs them back to back; the events bracket
    # the GPU time of the K steps).
    for i in range(warmup):
        decs[i % n_rep].run()
    torch.cuda.synchronize()
    K = max(1, steps)
    t_wall = time.perf_counter()
    torch.cuda._sleep(int(2.0e9 * (K * 40e-6 + 2e-3)))
    hip.hipEventRecord(outer[0], st)
    for i in range(K):
        decs[i % n_rep].run()
    hip.hipEventRecord(outer[1], st)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = elapsed_ms(hip, outer[0], outer[1])
    # Steady state, eager: at least 2,000 calls back to back the same way.
    n_ss = max(2000, 2 * n_rep)
    torch.cuda._sleep(int(2.0e9 * (n_ss * 40e-6 + 2e-3)))
    hip.hipEventRecord(outer[0], st)
    for i in range(n_ss):
        decs[i % n_rep].run()
    hip.hipEventRecord(outer[1], st)
    torch.cuda.synchronize()
    steady_ms = elapsed_ms(hip, outer[0], outer[1]) / n_ss
    # Steady state, graph: one HIP graph holding a step per input copy, replayed back to
    # back (at least 2,000 steps).
    big = csa2.capture_graph(decs)
    big.replay()
    torch.cuda.synchronize()
    n_big = max(1, math.ceil(2000 / n_rep))
    torch.cuda._sleep(int(2.0e9 * (n_big * 2e-5 + 2e-3)))
    hip.hipEventRecord(outer[0], st)
    for _ in range(n_big):
        big.replay()
    hip.hipEventRecord(outer[1], st)
    torch.cuda.synchronize()
    graph_ms = elapsed_ms(hip, outer[0], outer[1]) / (n_big * n_rep)
    del big
    return {"dw": dw, "reps": reps, "steps": K, "total_ms": total_ms, "ms_per_step": total_ms / K,
            "rows_per_s": wl.num_rows * K / (total_ms * 1e-3),
            "stages_us_eager": stages, "step_latency_us": lat_us, "wall_s_timed": t_wall,
            "input_replicas": n_rep,
            "steady_state": {"ms_per_step": steady_ms, "rows_per_s": wl.num_rows / (steady_ms * 1e-3),
                             "steps": n_ss, "launch": "eager"},
            "steady_state_graph": {"ms_per_step": graph_ms, "rows_per_s": wl.num_rows / (graph_ms * 1e-3),
                                   "steps": n_big * n_rep, "graph_replays": n_big}}


def attention_ms(csa2, hip, wl, reps, launches: int) -> float:
    """csa2_sparse_attn (attention + merge kernels) alone over the input copies, on the
    selection of the first copy's decode."""
    import torch
    d0 = csa2.Decoder(*reps[0].decode_inputs(), k=wl.k, n_keep=wl.n_keep, sm_scale=wl.sm_scale)
    d0.run()
    torch.cuda.synchronize()
    out = torch.empty((wl.num_rows, 64, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((wl.num_rows, 64), dtype=torch.float32, device="cuda")
    ws = torch.empty((max(256, csa2.sparse_attn_workspace_size(reps[0].rg, wl.k)),), dtype=torch.uint8, device="cuda")
    fns = [lambda r=r: csa2.sparse_attn(r.rg, r.q, r.main_kv, d0.sel_idx, d0.n_sel, r.swa, r.swa_scale,
                                        wl.sm_scale, out=out, lse=lse, ws=ws) for r in reps]
    return graph_kernel_ms(hip, fns, launches)


def scan_ms(csa2, hip, wl, idx_copies, dw, launches: int) -> float:
    import torch
    scores = torch.empty((wl.num_rows, max(1, wl.max_entries)), dtype=torch.float32, device="cuda")
    fns = [lambda k=k: csa2.index_score(dw.rg, k, dw.q_idx, dw.w, scores=scores) for k in idx_copies]
    for f in fns:
        f()
    return graph_kernel_ms(hip, fns, launches)


def scan_bytes(wl) -> int:
    """Algorithmic bytes of one indexer-scan launch over every entry: 68 B per entry plus
    each row's 8 x 128 bf16 query and 8 fp32 weights."""
    return wl.total_entries * 68 + wl.num_rows * (8 * 128 * 2 + 8 * 4)


def attn_flops(wl) -> int:
    return wl.num_rows * 4 * 64 * (512 + 128) * 512


def attn_bytes(wl) -> int:
    return wl.num_rows * (512 * 288 + 128 * (512 + 4) + 64 * 512 * 2 + 64 * 512 * 4 + 64 * 4)


ROOF_LAUNCHES = 200    # launches per timed run of a roofline kernel (steady state)
BURST_LAUNCHES = 20    # a short burst, reported beside it


def scale_rooflines(csa2, hip, launches: int = ROOF_LAUNCHES):
    """Scan and attention on the 64 x 128K decode batch (one row per request), each timed
    over runs of `launches` back-to-back launches (the median of five runs); the scan is
    also timed over bursts of BURST_LAUNCHES."""
    import torch
    from synth import make_config
    from synth.device import upload
    wl = make_config(5)
    dw = upload(wl)
    idx2 = dw.idx_k.clone()          # two copies (570 MB) alternate: no launch finds its keys cached
    s_ms = scan_ms(csa2, hip, wl, [dw.idx_k, idx2], dw, launches=launches)
    s_burst = scan_ms(csa2, hip, wl, [dw.idx_k, idx2], dw, launches=BURST_LAUNCHES)
    del idx2
    sb = scan_bytes(wl)
    gbs = sb / (s_ms * 1e-3) / 1e9
    traffic, traffic_note = None, "no counter summary for the current scan sources"
    cs = read_counter_summary("scan_64x128k_counters.md")
    if cs.get("kernel_sources_sha256") == sources_digest(SCAN_SOURCES):
        try:
            traffic = int(float(cs["fetch_bytes_per_launch"]) + float(cs["write_bytes_per_launch"]))
            traffic_note = "rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, scaled by a plain copy kernel " \
                           "(profiles/scan_64x128k_counters.md)"
        except (KeyError, ValueError):
            pass
    # Plain streaming read of the same bytes (csa2_debug_stream_read over two alternating
    # copies of the keys): what the memory system delivers to a kernel that only reads.
    idx3 = dw.idx_k.clone()
    sink = torch.zeros((4,), dtype=torch.int32, device="cuda")
    r_ms = graph_kernel_ms(hip, [lambda t=t: csa2.debug_stream_read(t, sink) for t in (dw.idx_k, idx3)],
                           launches=launches)
    del idx3
    read_gbs = sb / (r_ms * 1e-3) / 1e9
    roof = {"kernel": "indexer scan (csa2_index_score: every entry of 64 requests x 65536 entries)",
            "workload": "long_128k_x64: 64 requests x 131072 tokens pooled to 65536 entries, 1 row each",
            "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": traffic, "traffic_note": traffic_note, "bytes_per_launch": sb, "us_per_launch": s_ms * 1e3,
            "launches_per_run": launches,
            "burst_us_per_launch": s_burst * 1e3, "burst_frac": sb / (s_burst * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "burst_launches": BURST_LAUNCHES,
            "plain_read_GBs": read_gbs, "frac_of_plain_read": gbs / read_gbs,
            "plain_read_note": "csa2_debug_stream_read (non-temporal 16-B loads, 16 KiB per workgroup) over the same "
                               "285 MB, two alternating copies, same timing"}
    # The 1M-context batch (4 requests x 1,048,576 entries, 285 MB of keys).
    w4 = make_config(4, scan_only=True)
    if w4.num_rows:
        d4 = upload(w4)
        i4 = d4.idx_k.clone()
        s4 = scan_ms(csa2, hip, w4, [d4.idx_k, i4], d4, launches=launches)
        roof["unpooled_1m_scan"] = {"us_per_launch": s4 * 1e3, "bytes_per_launch": scan_bytes(w4),
                                    "achieved_GBs": scan_bytes(w4) / (s4 * 1e-3) / 1e9,
                                    "frac": scan_bytes(w4) / (s4 * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del d4, i4, w4
        torch.cuda.empty_cache()
    # Attention on the same batch: 64 rows, selections from one decode.
    reps = [dw]
    a_ms = attention_ms(csa2, hip, wl, reps + replicate(dw, 2)[1:], launches=launches)
    fl = attn_flops(wl)
    tfs = fl / (a_ms * 1e-3) / 1e12
    ab = attn_bytes(wl)
    util = None
    ca = read_counter_summary("attn_64rows_counters.md")
    if ca.get("kernel_sources_sha256") == sources_digest(ATTN_SOURCES):
        try:
            util = float(ca["mfma_busy_frac"])
        except (KeyError, ValueError):
            pass
    aroof = {"kernel": "sparse attention (csa2_sparse_attn: attention + merge kernels), 64 rows",
             "bound": "mfma", "achieved": tfs, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": tfs / BF16_PEAK_TFLOPS, "flops_per_launch": fl, "us_per_launch": a_ms * 1e3,
             "hbm_GBs": ab / (a_ms * 1e-3) / 1e9, "bytes_per_launch": ab, "launches_per_run": launches,
             "mfma_busy_frac_counters": util}
    return roof, aroof


def reference_copy(hip):
    """A plain elementwise kernel of known traffic (reads and writes 256 MiB) that the
    memory counters are scaled by."""
    import torch
    src = torch.ones((64 << 20,), dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()


CLOCK_INTERVAL = 500   # reference ticks (10 ns) between clock samples: 5 us


def clock_trace(csa2, hip, launches_list=(20, ROOF_LAUNCHES)) -> dict:
    """Shader clock while the 64 x 128K scan, and a plain read of the same bytes, run
    back to back: csa2_debug_clock_trace samples the clock on a side stream that waits
    for the same spin kernel as the launches, so sampling starts with the first launch.
    Per kernel and run length: the mean clock over the run, over its first 1 ms and over
    its last 20 % (GHz), and the run's microseconds per launch."""
    import torch
    from synth import make_config
    from synth.device import upload
    wl = make_config(5)
    dw = upload(wl)
    idx2 = dw.idx_k.clone()
    scores = torch.empty((wl.num_rows, wl.max_entries), dtype=torch.float32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    kinds = {"scan": [lambda k=k: csa2.index_score(dw.rg, k, dw.q_idx, dw.w, scores=scores) for k in (dw.idx_k, idx2)],
             "plain_read": [lambda t=t: csa2.debug_stream_read(t, sink) for t in (dw.idx_k, idx2)]}
    main_st, side = torch.cuda.current_stream(), torch.cuda.Stream()
    ev = make_events(hip, 2)
    st = ctypes.c_void_p(main_st.cuda_stream)
    res = {}
    for name, fns in kinds.items():
        for f in fns:
            f()
        torch.cuda.synchronize()
        for n in launches_list:
            samples = min(60000, int(n * 60e-6 / (CLOCK_INTERVAL * 1e-8)) + 40)
            buf = torch.zeros(2 * samples, dtype=torch.int64, device="cuda")
            torch.cuda._sleep(int(2.0e9 * (n * 60e-6 + 3e-3)))
            go = torch.cuda.Event()
            go.record(main_st)
            side.wait_event(go)
            with torch.cuda.stream(side):
                csa2.debug_clock_trace(buf, samples, CLOCK_INTERVAL)
            hip.hipEventRecord(ev[0], st)
            for i in range(n):
                fns[i % len(fns)]()
            hip.hipEventRecord(ev[1], st)
            torch.cuda.synchronize()
            us = elapsed_ms(hip, ev[0], ev[1]) * 1e3
            v = buf.cpu().numpy().astype(np.float64)
            t, r = v[0::2], (v[1::2] - v[1]) / 100.0            # r in microseconds from the first sample
            def ghz(lo, hi):
                i = np.nonzero((r >= lo) & (r <= hi))[0]
                return float(0.1 * (t[i[-1]] - t[i[0]]) / ((r[i[-1]] - r[i[0]]) * 100.0)) if len(i) > 1 else None
            res[f"{name}_{n}"] = {"launches": n, "us_per_launch": us / n, "run_us": us,
                                  "clock_GHz_run": ghz(0.0, us), "clock_GHz_first_1ms": ghz(0.0, min(1000.0, us)),
                                  "clock_GHz_last_20pct": ghz(0.8 * us, us)}
    # The sampler alone (no load).
    buf = torch.zeros(2 * 200, dtype=torch.int64, device="cuda")
    csa2.debug_clock_trace(buf, 200, CLOCK_INTERVAL)
    torch.cuda.synchronize()
    v = buf.cpu().numpy().astype(np.float64)
    res["idle"] = {"clock_GHz": float(0.1 * (v[-2] - v[0]) / (v[-1] - v[1]))}
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=1, help="headline workload id (default 1: 128K-context decode)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-scale", action="store_true", help="skip the 64 x 128K roofline loops")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads")
    ap.add_argument("--profile-scale", action="store_true",
                    help="only the 64 x 128K scan/attention loops and the reference copy (for counter runs)")
    ap.add_argument("--clock-trace", action="store_true",
                    help="only the shader clock during 20- and 200-launch runs of the scan and the plain read")
    ap.add_argument("--launches", type=int, default=ROOF_LAUNCHES,
                    help="back-to-back launches per timed run of a roofline kernel")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import sparse_decode_attention_csa2_amd as csa2
    from synth import make_config

    if not os.path.exists(csa2.LIB_PATH):
        from __graft_entry__ import build
        build()
    torch.cuda.set_device(0)
    hip = _hip()

    if args.clock_trace:
        print(json.dumps({"clock_trace": clock_trace(csa2, hip)}), flush=True)
        return 0
    if args.profile_scale:
        roof, aroof = scale_rooflines(csa2, hip, launches=args.launches)
        reference_copy(hip)
        print(json.dumps({"roofline": roof, "attention_roofline": aroof}), flush=True)
        return 0

    K, W = args.steps, args.warmup
    wl = make_config(args.config)
    m = measure_decode(csa2, hip, wl, K, W)
    reps = m["reps"]
    # Per-kernel rooflines at the headline workload: the scan and attention alone.
    s_ms = scan_ms(csa2, hip, wl, [r.idx_k for r in reps], reps[0], launches=max(ROOF_LAUNCHES, len(reps)))
    a_ms = attention_ms(csa2, hip, wl, reps, launches=max(ROOF_LAUNCHES, len(reps)))
    sb = scan_bytes(wl)
    head = {
        "scan": {"us_per_launch": s_ms * 1e3, "bytes_per_launch": sb,
                 "achieved_GBs": sb / (s_ms * 1e-3) / 1e9, "frac_of_hbm_peak": sb / (s_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "attention": {"us_per_launch": a_ms * 1e3, "flops_per_launch": attn_flops(wl),
                      "achieved_TFLOPs": attn_flops(wl) / (a_ms * 1e-3) / 1e12,
                      "frac_of_bf16_peak": attn_flops(wl) / (a_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                      "bytes_per_launch": attn_bytes(wl)},
    }
    del reps, m["reps"], m["dw"]
    torch.cuda.empty_cache()

    res = {
        "metric": "decode query-rows/s + indexer-scan HBM GB/s (% of peak) at 128K ctx, top-512",
        "value": m["rows_per_s"],
        "unit": "query-rows/s",
        "n_gpus": 1, "steps": m["steps"], "warmup": W, "ms_per_step": m["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4/fp8 in, bf16 mfma, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.num_requests} request(s) x {wl.num_rows // max(1, wl.num_requests)} "
                               f"row(s), {wl.total_entries} entries, top-{wl.k}, keep {wl.n_keep}+newest blocks, "
                               f"128-token FP8 window",
                   "requests": wl.num_requests, "rows": wl.num_rows, "entries": wl.total_entries,
                   "input_replicas": m["input_replicas"]},
        "launch": "exactly --steps csa2_decode calls (one launch chain each), rotating over the input replicas, "
                  "enqueued behind a spin kernel and timed between HIP events on the stream",
        "steady_state": m["steady_state"],
        "steady_state_graph": m["steady_state_graph"],
        "stages_us_eager": m["stages_us_eager"],
        "step_latency_us": m["step_latency_us"],
        "kernels_headline": head,
        "step_bytes": step_bytes(wl),
        "step_GBs": step_bytes(wl) / (m["ms_per_step"] * 1e-3) / 1e9,
        "step_frac_of_hbm_peak": step_bytes(wl) / (m["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "wall_s_timed": m["wall_s_timed"],
    }
    if not args.no_scale:
        roof, aroof = scale_rooflines(csa2, hip, launches=args.launches)
        res["roofline"] = roof
        res["attention_roofline"] = aroof
        torch.cuda.empty_cache()
    if not args.no_configs:
        from synth import to_paged, verify_row_len
        per = {}

        def paged_rowlen(i):
            w = make_config(i)
            w.row_len = verify_row_len(w)
            w = to_paged(w)
            w.name = w.name.replace("_paged", "_paged_rowlen")
            return w

        # The other decode workloads, then two served shapes: the headline over paged
        # pools, and the verify batch over paged pools with per-row visible lengths.
        # The MXFP8 Q/P route of the attention on the headline and 64-row workloads.
        # The candidate-only scan (scan_mode 1: coarse stage first, then only the kept
        # blocks' keys) on the headline, 64 x 128K, 1M-context and verify workloads.
        cases = [(0, 0, lambda i=i: make_config(i)) for i in (0, 2, 3, 4, 5) if i != args.config]
        cases += [(0, 0, lambda: to_paged(make_config(args.config))), (0, 0, lambda: paged_rowlen(3))]
        cases += [(csa2.QP_MXFP8, 0, lambda: make_config(args.config)), (csa2.QP_MXFP8, 0, lambda: make_config(5))]
        cases += [(0, 1, lambda i=i: make_config(i)) for i in (args.config, 5, 4, 3)]
        for route, smode, mk in cases:
            w = mk()
            mi = measure_decode(csa2, hip, w, steps=max(64, min(K, 400)), warmup=8, qp_route=route,
                                scan_mode=smode)
            name = w.name + ("_mxfp8" if route == csa2.QP_MXFP8 else "") + ("_candidate_scan" if smode else "")
            gbs = step_bytes(w) / (mi["ms_per_step"] * 1e-3) / 1e9
            per[name] = {"requests": w.num_requests, "rows": w.num_rows, "entries": w.total_entries,
                           "paged": w.page_table is not None, "row_len": w.row_len is not None,
                           "qp_route": "mxfp8" if route == csa2.QP_MXFP8 else "bf16",
                           "scan_mode": smode,
                           "rows_per_s": mi["rows_per_s"], "ms_per_step": mi["ms_per_step"],
                           "step_bytes": step_bytes(w), "step_GBs": gbs, "step_frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
                           "step_latency_us": mi["step_latency_us"], "steady_state": mi["steady_state"],
                           "steady_state_graph": mi["steady_state_graph"],
                           "stages_us_eager": mi["stages_us_eager"], "input_replicas": mi["input_replicas"]}
            del mi, w
            torch.cuda.empty_cache()
        res["per_config"] = per
        res["cache_write"] = cache_write_timing(csa2, hip)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
