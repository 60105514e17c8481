"""End-to-end parity of csa2_decode against the oracle on the five decode workloads and
on edge cases (needs an MI355X)."""
import os
import sys
import time

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
from synth import to_paged, make_config, make_workload
from synth.device import upload

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def csa2():
    import sparse_decode_attention_csa2_amd as m
    if not os.path.exists(m.LIB_PATH):
        pytest.fail("libcsa2.so missing: the HIP path must be built before GPU tests")
    m.load_library()
    return m


def run_decode(csa2, wl, **kw):
    dw = upload(wl)
    d = csa2.Decoder(*dw.decode_inputs(), k=kw.pop("k", wl.k), n_keep=kw.pop("n_keep", wl.n_keep),
                     keep_newest=bool(kw.pop("keep_newest", wl.keep_newest)), sm_scale=wl.sm_scale, **kw)
    d.run()
    torch.cuda.synchronize()
    return dict(out=d.out.cpu().numpy(), lse=d.lse.cpu().numpy(), sel=d.sel_idx.cpu().numpy(),
                n_sel=d.n_sel.cpu().numpy(), kept=d.kept.cpu().numpy(), n_kept=d.n_kept.cpu().numpy(),
                scores=d.scores.cpu().numpy())


def judge(wl, got, refs, rows=None, k=None, n_keep=None):
    rows = list(range(wl.num_rows)) if rows is None else rows
    reports = []
    for r, ref in zip(rows, refs):
        rep = parity.check_row(wl, r, ref, got["kept"][r, :got["n_kept"][r]], got["sel"][r, :got["n_sel"][r]],
                               got["out"][r], got["lse"][r], k=k, n_keep=n_keep)
        reports.append(rep)
    bad = [rp for rp in reports if not rp["ok"]]
    worst = max((rp["attn_rel_own"] for rp in reports), default=0.0)
    _log(f"  rows {len(reports)}: sets equal {sum(rp['set_equal'] for rp in reports)}, "
         f"kept equal {sum(rp.get('kept_equal', True) for rp in reports)}, worst attn rel {worst:.2e}")
    assert not bad, "; ".join(f"row {rp['row']}: {' | '.join(rp['msgs'])}" for rp in bad[:5])
    return reports


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_decode_config_matches_oracle(csa2, cfg):
    t0 = time.time()
    wl = make_config(cfg)
    _log(f"config {cfg} ({wl.name}): {wl.num_requests} requests, {wl.num_rows} rows, "
         f"{wl.total_entries} entries (generated in {time.time() - t0:.1f}s)")
    got = run_decode(csa2, wl)
    _log(f"  decode done; oracle ...")
    refs = oracle.decode(wl)
    # Index scores (diagnostic bound: fp32 vs fp64 within 1e-5 of the mean score).
    for b in range(wl.num_requests):
        r0 = int(wl.row_off[b])
        n = wl.n_entries(b)
        ref = refs[r0]["scores"]
        err = np.abs(got["scores"][r0, :n] - ref).max() / np.abs(ref).mean()
        assert err <= 1e-5, f"request {b}: score error {err:.3g}"
    judge(wl, got, refs)
    _log(f"  config {cfg} ok in {time.time() - t0:.1f}s")


def test_decode_candidate_only_scan_matches_full_scan(csa2):
    wl = make_config(3)
    full = run_decode(csa2, wl)
    cand = run_decode(csa2, wl, scan_mode=1)
    assert np.array_equal(full["sel"], cand["sel"]) and np.array_equal(full["n_sel"], cand["n_sel"])
    assert np.array_equal(full["kept"], cand["kept"])
    assert np.array_equal(full["out"], cand["out"]) and np.array_equal(full["lse"], cand["lse"])


def test_decode_is_deterministic(csa2):
    wl = make_config(2)
    a = run_decode(csa2, wl)
    b = run_decode(csa2, wl)
    for key in ("out", "lse", "sel", "kept", "scores"):
        assert np.array_equal(a[key], b[key], equal_nan=True), key


def test_decode_edge_workloads(csa2):
    # Empty request, single entry, partial blocks, nb <= 64 (coarse stage keeps all),
    # nb just above 64, N < k, windows of 0..128 tokens, several rows per request.
    lens = [0, 1, 63, 64, 65, 511, 513, 64 * 64, 64 * 64 + 1, 64 * 65, 64 * 65 + 63, 20000]
    swa = [0, 1, 128, 5, 0, 128, 77, 128, 128, 1, 128, 128]
    rows = [1, 1, 2, 1, 1, 3, 1, 1, 6, 1, 1, 2]
    wl = make_workload("edge", 99, lens, rows_per_req=rows, n_needles=4, swa_len=swa)
    _log(f"edge workload: {len(lens)} requests, {wl.num_rows} rows")
    got = run_decode(csa2, wl)
    refs = oracle.decode(wl)
    judge(wl, got, refs)
    r_empty = 0
    assert got["n_sel"][r_empty] == 0 and np.all(np.isneginf(got["lse"][r_empty]))
    assert np.all(got["out"][r_empty] == 0)


@pytest.mark.parametrize("k,n_keep,newest", [(100, 10, True), (2048, 128, True), (512, 64, False), (1, 1, True)])
def test_decode_parameters(csa2, k, n_keep, newest):
    wl = make_workload("params", 7 + k, [64 * 300 + 3, 4096, 64 * 129], rows_per_req=[1, 2, 1], n_needles=16)
    _log(f"decode k {k} n_keep {n_keep} newest {newest}")
    got = run_decode(csa2, wl, k=k, n_keep=n_keep, keep_newest=newest)
    refs = oracle.decode(wl, k=k, n_keep=n_keep, keep_newest=int(newest))
    judge(wl, got, refs, k=k, n_keep=n_keep)


def test_decode_keep_all_is_dense_attention(csa2):
    # k >= N and n_keep >= nb: every entry is selected and the result is dense attention
    # over all entries plus the window.
    wl = make_workload("dense", 17, [2000, 64 * 100], rows_per_req=[2, 1], n_needles=0)
    got = run_decode(csa2, wl, k=2048, n_keep=128)
    for r in range(wl.num_rows):
        b = int(wl.row_req[r])
        n = wl.n_entries(b)
        if n <= 2048:
            assert got["sel"][r, :got["n_sel"][r]].tolist() == list(range(n))
            ro, rl = oracle.joint_attention(oracle.bf16_value(wl.q[r]), oracle.row_keys(wl, r, np.arange(n)),
                                            wl.sm_scale)
            rel, dl = parity.attn_error(got["out"][r], got["lse"][r], ro, rl)
            assert rel <= parity.ATTN_REL and dl <= parity.LSE_ABS


def test_decode_beyond_lds_block_buffer(csa2):
    # A request with more 64-entry blocks than the select's LDS key buffer holds (16,384):
    # its coarse stage ranks straight from global memory, while the shorter request of
    # the same launch (blk_ld above the buffer too) takes the LDS path without prefetch.
    lens = [64 * 16384 + 70, 64 * 300 + 5]
    wl = make_workload("beyond", 23, lens, rows_per_req=[1, 2], n_needles=16)
    _log(f"decode beyond the LDS block buffer: lengths {lens}")
    got = run_decode(csa2, wl)
    refs = oracle.decode(wl)
    judge(wl, got, refs)
    dw = upload(wl)
    kept, n_kept, _ = csa2.block_filter(dw.rg, dw.blk_sum, dw.q_idx, dw.w, n_keep=64)
    assert np.array_equal(kept.cpu().numpy(), got["kept"]) and np.array_equal(n_kept.cpu().numpy(), got["n_kept"])


def test_request_without_summaries_in_the_pool(csa2):
    # block_off is clamped to the summary pool: a request whose summaries start at its end
    # has no blocks to rank (nothing kept, nothing selected: attention over its window
    # only), and the other requests are unaffected.  Three rows in request 0 make the one
    # scan launch score each workgroup's own blocks, the path that clamps this case.
    wl = make_workload("noblk", 51, [64 * 40 + 9, 64 * 12 + 5], rows_per_req=[3, 1], n_needles=4)
    _log("request 1 with no summaries in the pool")
    ref = run_decode(csa2, wl, k=256, n_keep=16)
    end0 = int(wl.block_off[1])
    wl.block_off = wl.block_off.copy()
    wl.block_off[2] = end0
    wl.blk_sum = wl.blk_sum[:end0].copy()   # the pool ends where request 1's summaries would start
    got = run_decode(csa2, wl, k=256, n_keep=16)
    for key in ("out", "lse", "sel", "kept", "n_sel", "n_kept"):
        a, b = np.ascontiguousarray(got[key][:3]), np.ascontiguousarray(ref[key][:3])
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b), key
    assert got["n_kept"][3] == 0 and got["n_sel"][3] == 0
    assert (got["sel"][3] == -1).all() and (got["kept"][3] == -1).all()
    assert np.isfinite(got["out"][3]).all() and np.isfinite(got["lse"][3]).all()


def test_contiguous_key_reads_with_ragged_tails(csa2):
    # Eight one-row requests, long enough (ceil(max_entries / 256) x 8 >= 8,192 tiles) that
    # the decode's one scan launch runs 4 chunks per wave, where each wave reads its
    # 64-entry chunk of keys as one contiguous run and regroups it through LDS.  The
    # lengths leave partial chunks and workgroups at every request's end.  The decode's
    # scores and the entry-only scan's equal a direct-load scan's bit for bit, and rows are judged
    # against the oracle.  The entry-only scan of these contiguous pools takes the
    # contiguous reads too, so the direct-load reference is the scan over the same
    # workload in paged pools (bit-exact with contiguous ones).
    lens = [262144 + 37, 262144 - 1, 200003, 131072 + 64 * 5 + 1, 70001, 4097, 65, 262144 - 200]
    tiles1, iters = -(-max(lens) // 256), 1
    while iters < 4 and tiles1 * len(lens) >= 2048 * 2 * iters:
        iters *= 2
    assert iters == 4
    wl = make_workload("ldsk", 52, lens, rows_per_req=1, n_needles=8)
    _log(f"contiguous key reads, ragged lengths {lens}")
    got = run_decode(csa2, wl)
    dw = upload(wl)
    flat = csa2.index_score(dw.rg, dw.idx_k, dw.q_idx, dw.w).cpu().numpy()
    pw = upload(to_paged(wl))
    ref = csa2.index_score(pw.rg, pw.idx_k, pw.q_idx, pw.w).cpu().numpy()
    for r, n in enumerate(lens):
        assert np.array_equal(got["scores"][r, :n].view(np.uint32), ref[r, :n].view(np.uint32)), f"row {r}"
        assert np.array_equal(flat[r, :n].view(np.uint32), ref[r, :n].view(np.uint32)), f"row {r}"
    rows = [0, 3, 6]
    judge(wl, got, oracle.decode(wl, rows=rows), rows=rows)


def test_bench_scale_batches_on_sampled_rows(csa2):
    # The two 285 MB batches bench.py times the scan on (64 x 65,536 entries, 4 chunks per
    # wave; 4 x 1,048,576 entries), in the launch configuration it times: the full-scan
    # scores of sampled requests, and whole decode rows of the 64-request batch.
    from synth import make_config as mk
    wl = mk(5)
    _log(f"64 x 128K batch: {wl.total_entries} entries")
    dw = upload(wl)
    scores = csa2.index_score(dw.rg, dw.idx_k, dw.q_idx, dw.w).cpu().numpy()
    for b in (0, 17, 42, 63):
        ref = oracle.request_scores(wl, b)[0]
        err = np.abs(scores[b, :wl.n_entries(b)] - ref).max() / np.abs(ref).mean()
        assert err <= 1e-5, f"request {b}: score error {err:.3g}"
    rows = [0, 31, 63]
    got = run_decode(csa2, wl)
    refs = oracle.decode(wl, rows=rows)
    judge(wl, got, refs, rows=rows)
    del dw, wl
    torch.cuda.empty_cache()
    w4 = mk(4, scan_only=True)
    d4 = upload(w4)
    s4 = csa2.index_score(d4.rg, d4.idx_k, d4.q_idx, d4.w).cpu().numpy()
    for b in (0, 3):
        ref = oracle.request_scores(w4, b)[0]
        err = np.abs(s4[b, :w4.n_entries(b)] - ref).max() / np.abs(ref).mean()
        assert err <= 1e-5, f"1M request {b}: score error {err:.3g}"


@pytest.mark.parametrize("n_keep", [1, 4])
def test_sliced_coarse_stage_with_few_kept_blocks(csa2, n_keep):
    # Rows with more than 4,096 blocks rank 1,024-block slices first and then the slices'
    # candidates (n_slices x n_keep of them).  With n_keep 1 or 4 those candidates are far
    # fewer than one gather batch of the select, whose validity check then runs over
    # slots past the last slice's count.  Kept blocks equal the one-level block filter's
    # and rows are judged against the oracle.
    lens = [64 * 5000 + 17, 64 * 4500 + 3]
    wl = make_workload("sliced", 61 + n_keep, lens, rows_per_req=1, n_needles=8)
    _log(f"sliced coarse stage, n_keep {n_keep}, lengths {lens}")
    got = run_decode(csa2, wl, n_keep=n_keep)
    judge(wl, got, oracle.decode(wl, n_keep=n_keep), n_keep=n_keep)
    dw = upload(wl)
    kept, n_kept, _ = csa2.block_filter(dw.rg, dw.blk_sum, dw.q_idx, dw.w, n_keep=n_keep)
    assert np.array_equal(kept.cpu().numpy(), got["kept"]) and np.array_equal(n_kept.cpu().numpy(), got["n_kept"])


def test_decode_with_workspace_at_the_end_of_an_allocation(csa2):
    # The workspace is exactly csa2_decode_workspace_size bytes and ends where its
    # allocation ends (a 2 MiB multiple, which the caching allocator hands out whole);
    # its last buffer holds the sliced coarse stage's per-slice counts.
    wl = make_workload("exactws", 71, [64 * 5000 + 17], rows_per_req=1, n_needles=8)
    dw = upload(wl)
    d = csa2.Decoder(*dw.decode_inputs(), k=wl.k, n_keep=1, sm_scale=wl.sm_scale)
    n = d.ws_bytes
    total = -(-n // (2 << 20)) * (2 << 20)
    big = torch.empty((total,), dtype=torch.uint8, device="cuda")
    d.ws = big[total - n:]
    assert d.ws.data_ptr() % 256 == 0 and d.ws.numel() == n
    _log(f"decode with a {n}-byte workspace at the end of a {total}-byte allocation")
    d.run()
    torch.cuda.synchronize()
    got = dict(out=d.out.cpu().numpy(), lse=d.lse.cpu().numpy(), sel=d.sel_idx.cpu().numpy(),
               n_sel=d.n_sel.cpu().numpy(), kept=d.kept.cpu().numpy(), n_kept=d.n_kept.cpu().numpy())
    judge(wl, got, oracle.decode(wl, n_keep=1), n_keep=1)


def test_entry_scan_long_workgroups_ragged(csa2):
    # The entry-only scan over contiguous pools sizes its workgroups so that the grid is
    # one round of five per CU: here 13 chunks (832 entries) per wave, 3,328-entry
    # workgroups (a multiple of neither 2,048 nor a power of two).  Lengths that are not
    # multiples of 64 leave partial workgroups and chunks at every request's end.  Scores
    # equal the direct-load scan's (the same workload over paged pools) bit for bit, and
    # sampled requests are judged against the oracle.
    lens = [524288 + 37, 524288 - 1, 400003, 262144 + 64 * 5 + 1, 140001, 4097, 65, 524288 - 200]
    chunks = -(-max(lens) // 64)
    per_req = 5 * 256 // len(lens)
    iters = min(max(-(-chunks // (4 * per_req)), 4), 14)
    assert iters == 13
    wl = make_workload("ldsk8", 53, lens, rows_per_req=1, n_needles=8, scan_only=True)
    _log(f"entry-only scan at {iters} chunks per wave, ragged lengths {lens}")
    dw = upload(wl)
    flat = csa2.index_score(dw.rg, dw.idx_k, dw.q_idx, dw.w).cpu().numpy()
    del dw
    pw = upload(to_paged(wl))
    ref = csa2.index_score(pw.rg, pw.idx_k, pw.q_idx, pw.w).cpu().numpy()
    del pw
    torch.cuda.empty_cache()
    for r, n in enumerate(lens):
        assert np.array_equal(flat[r, :n].view(np.uint32), ref[r, :n].view(np.uint32)), f"row {r}"
    for b in (2, 6, 7):
        want = oracle.request_scores(wl, b)[0]
        err = np.abs(flat[b, :lens[b]] - want).max() / np.abs(want).mean()
        assert err <= 1e-5, f"request {b}: score error {err:.3g}"


def test_decode_bits_do_not_depend_on_the_grid(csa2):
    # Same inputs, different workgroup counts: a larger host-side max_entries (still within
    # the pools) changes the scan's workgroup size and count and the select's gather range;
    # every output stays identical bit for bit.
    wl = make_config(2)
    dw = upload(wl)
    outs = []
    for scale in (1, 4):
        rg = dw.rg
        big = type(rg)(**{f: getattr(rg, f) for f in rg.__dataclass_fields__})
        big.max_entries = min(rg.total_entries, rg.max_entries * scale)
        d = csa2.Decoder(big, *dw.decode_inputs()[1:], k=wl.k, n_keep=wl.n_keep, sm_scale=wl.sm_scale)
        d.run()
        torch.cuda.synchronize()
        _log(f"max_entries {big.max_entries}: workspace {d.ws_bytes} bytes")
        outs.append({k: getattr(d, k).cpu().numpy() for k in ("out", "lse", "sel_idx", "n_sel", "kept", "n_kept")})
        sc = d.scores.cpu().numpy()
        outs[-1]["scores"] = np.concatenate([sc[r, :wl.n_entries(int(wl.row_req[r]))] for r in range(wl.num_rows)])
    for key in outs[0]:
        a, b = outs[0][key], outs[1][key]
        if a.dtype == np.float32:
            a, b = a.view(np.uint32), b.view(np.uint32)
        assert np.array_equal(a, b), key


def _judge_candidate_scores(wl, got, refs, rows):
    # In the candidate-only scan only the kept blocks' entries the row sees are scored.
    for r, ref in zip(rows, refs):
        nk = int(got["n_kept"][r])
        n = wl.n_entries(int(wl.row_req[r]))
        pos = np.concatenate([np.arange(64 * j, min(64 * j + 64, n)) for j in got["kept"][r, :nk]])
        want = ref["scores"][pos]
        err = np.abs(got["scores"][r, pos] - want).max() / np.abs(want).mean()
        assert err <= 1e-5, f"row {r}: candidate score error {err:.3g}"


@pytest.mark.parametrize("cfg", [1, 4])
def test_candidate_only_scan_matches_oracle(csa2, cfg):
    # scan_mode 1: the coarse stage runs first and only the kept blocks' keys are
    # scored; the selected set is the full scan's by construction, and the whole row is
    # judged against the oracle (128K context, and the 1M-context batch).
    wl = make_config(cfg)
    _log(f"candidate-only scan, config {cfg} ({wl.name}): {wl.num_rows} rows, {wl.total_entries} entries")
    got = run_decode(csa2, wl, scan_mode=1)
    rows = list(range(wl.num_rows))
    refs = oracle.decode(wl)
    judge(wl, got, refs)
    _judge_candidate_scores(wl, got, refs, rows)


def test_candidate_only_scan_on_sampled_64x128k_rows(csa2):
    # The 64 x 128K batch bench.py times in candidate-only mode: sampled rows against the
    # oracle, and every row's selection equal to the full scan's.
    wl = make_config(5)
    _log(f"candidate-only scan, 64 x 128K batch: {wl.total_entries} entries")
    got = run_decode(csa2, wl, scan_mode=1)
    full = run_decode(csa2, wl)
    assert np.array_equal(got["kept"], full["kept"]) and np.array_equal(got["n_kept"], full["n_kept"])
    assert np.array_equal(got["sel"], full["sel"]) and np.array_equal(got["n_sel"], full["n_sel"])
    assert np.array_equal(got["out"].view(np.uint32), full["out"].view(np.uint32))
    rows = [0, 17, 40, 63]
    refs = oracle.decode(wl, rows=rows)
    judge(wl, got, refs, rows=rows)
    _judge_candidate_scores(wl, got, refs, rows)
