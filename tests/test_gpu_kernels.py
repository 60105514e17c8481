"""Per-kernel parity of the HIP path against the oracle (needs an MI355X)."""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
from synth import make_workload
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


def _same_bits(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(nan | (a.view(np.uint32) == b.view(np.uint32))))


# ----------------------------------------------------------------------------------
# Dequantisation: bit-exact over exhaustive tables.
# ----------------------------------------------------------------------------------

def test_dequant_fp4_main_exhaustive(csa2):
    _log("dequant main: 256 scale codes x 256 code bytes")
    rec = np.zeros((256, 288), dtype=np.uint8)
    rec[:, :256] = np.arange(256, dtype=np.uint8)[None, :]     # every (low, high) nibble pair
    rec[:, 256:] = np.arange(256, dtype=np.uint8)[:, None]     # record i: every scale = code i
    got = csa2.debug_dequant(csa2.DQ_MAIN, torch.from_numpy(rec).cuda()).cpu().numpy()
    ref = oracle.dequant_main(rec).astype(np.float32)
    assert _same_bits(got, ref)


def test_dequant_fp4_idx_exhaustive(csa2):
    _log("dequant idx: 256 scale codes x all nibble pairs")
    rng = np.random.default_rng(0)
    rec = np.zeros((4 * 256, 68), dtype=np.uint8)
    for part in range(4):   # bytes 0..63 of the 4 parts cover all 256 byte values
        rec[part * 256:(part + 1) * 256, :64] = (np.arange(64) + 64 * part).astype(np.uint8)[None, :]
    rec[:, 64:] = np.tile(np.arange(256, dtype=np.uint8), 4)[:, None]
    rec[::7, 64:] = rng.integers(0, 256, size=(rec[::7].shape[0], 4), dtype=np.uint8)
    got = csa2.debug_dequant(csa2.DQ_IDX, torch.from_numpy(rec).cuda()).cpu().numpy()
    ref = oracle.dequant_idx(rec).astype(np.float32)
    assert _same_bits(got, ref)


def test_dequant_e4m3_exhaustive(csa2):
    _log("dequant e4m3: 256 codes x scale set")
    scales = np.array([1.0, 0.5, 448.0 ** -1, 3.7e-3, 1.7e-2, 2.0 ** -20, 123.456, 1e-30], dtype=np.float32)
    rec = np.zeros((scales.size, 512), dtype=np.uint8)
    rec[:, :256] = np.arange(256, dtype=np.uint8)
    rec[:, 256:] = np.arange(255, -1, -1, dtype=np.uint8)
    got = csa2.debug_dequant(csa2.DQ_SWA, torch.from_numpy(rec).cuda(), torch.from_numpy(scales).cuda())
    ref = oracle.dequant_swa(rec, scales).astype(np.float32)      # fp64 product rounded once
    assert _same_bits(got.cpu().numpy(), ref)


# ----------------------------------------------------------------------------------
# Indexer scan and block scores.
# ----------------------------------------------------------------------------------

def _score_close(got, ref, name):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    scale = max(1e-30, float(np.abs(ref).mean()))
    err = float(np.abs(got - ref).max()) / scale if ref.size else 0.0
    assert err <= 1e-5, f"{name}: max error {err:.3g} of the mean score"
    return err


@pytest.mark.parametrize("rows", [1, 2, 6, 16])
def test_index_score_matches_oracle(csa2, rows):
    lens = [1, 63, 64, 65, 300, 1000, 4097][: (7 if rows < 16 else 3)]
    _log(f"index scan: rows/request {rows}, lengths {lens}")
    wl = make_workload("scan", 10 + rows, lens, rows_per_req=rows, n_needles=3)
    dw = upload(wl)
    scores = csa2.index_score(dw.rg, dw.idx_k, dw.q_idx, dw.w).cpu().numpy()
    for b in range(wl.num_requests):
        ref = oracle.request_scores(wl, b)
        n = wl.n_entries(b)
        for j, r in enumerate(range(int(wl.row_off[b]), int(wl.row_off[b + 1]))):
            _score_close(scores[r, :n], ref[j], f"request {b} row {r}")
            assert np.all(np.isnan(scores[r, n:])), "scores beyond the request's entries were written"


@pytest.mark.parametrize("rows", [1, 3, 6, 16])
def test_index_score_multi_chunk_waves(csa2, rows):
    # Requests long enough that each wave walks several 64-entry chunks (the launch
    # heuristic doubles chunks per wave at 4 x 262144 entries), with ragged tails, for
    # every query-row grouping (score staging per workgroup and per chunk).
    lens = [262144, 262144 - 37, 200001, 262144]
    _log(f"index scan, multi-chunk waves: rows/request {rows}, lengths {lens}")
    wl = make_workload("scanlong", 40 + rows, lens, rows_per_req=rows, n_needles=3, scan_only=True)
    dw = upload(wl)
    scores = csa2.index_score(dw.rg, dw.idx_k, dw.q_idx, dw.w).cpu().numpy()
    for b in range(wl.num_requests):
        ref = oracle.request_scores(wl, b)
        n = wl.n_entries(b)
        for j, r in enumerate(range(int(wl.row_off[b]), int(wl.row_off[b + 1]))):
            _score_close(scores[r, :n], ref[j], f"request {b} row {r}")
            assert np.all(np.isnan(scores[r, n:])), "scores beyond the request's entries were written"


def test_block_filter_matches_oracle(csa2):
    lens = [64 * 64, 64 * 64 + 1, 64 * 100 + 17, 64 * 300, 5000, 10]
    _log(f"block filter: lengths {lens}")
    wl = make_workload("blk", 21, lens, rows_per_req=[1, 2, 1, 6, 1, 1], n_needles=8)
    dw = upload(wl)
    kept, n_kept, bsc = csa2.block_filter(dw.rg, dw.blk_sum, dw.q_idx, dw.w, n_keep=64)
    kept, n_kept, bsc = kept.cpu().numpy(), n_kept.cpu().numpy(), bsc.cpu().numpy()
    for r in range(wl.num_rows):
        ref_bs = oracle.block_scores_row(wl, r)
        nb = ref_bs.size
        _score_close(bsc[r, :nb], ref_bs, f"row {r} block scores")
        ref_kept = oracle.keep_blocks(ref_bs, 64)
        got = kept[r, :n_kept[r]]
        assert np.all(kept[r, n_kept[r]:] == -1)
        if not np.array_equal(got, ref_kept):
            ok, msg = parity.band_ok(sorted(set(got.tolist()) ^ set(ref_kept.tolist())), lambda j: ref_bs[j],
                                     parity.kth_best(ref_bs, 64), parity.SET_REL)
            assert ok, f"row {r}: {msg}"


@pytest.mark.parametrize("n_keep,newest", [(64, True), (64, False), (3, True), (128, True)])
def test_block_select_exact_with_ties(csa2, n_keep, newest):
    # Summaries built so that block scores tie exactly in fp32 and fp64: only a few
    # distinct summary vectors, all with small-integer dot products.
    _log(f"block select ties: n_keep {n_keep} newest {newest}")
    wl = make_workload("ties", 5, [64 * 200, 64 * 77 + 5], rows_per_req=1, n_needles=0)
    rng = np.random.default_rng(1)
    base = rng.integers(-2, 3, size=(4, 128)).astype(np.float32)
    pick = rng.integers(0, 4, size=wl.blk_sum.shape[0])
    wl.blk_sum[:] = (base[pick].view(np.uint32) >> 16).astype(np.uint16)
    wl.q_idx[:] = (np.ones((wl.num_rows, 8, 128), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wl.w[:] = 1.0
    dw = upload(wl)
    kept, n_kept, _ = csa2.block_filter(dw.rg, dw.blk_sum, dw.q_idx, dw.w, n_keep=n_keep, keep_newest=newest)
    kept, n_kept = kept.cpu().numpy(), n_kept.cpu().numpy()
    for r in range(wl.num_rows):
        ref = oracle.keep_blocks(oracle.block_scores_row(wl, r), n_keep, newest)
        assert kept[r, :n_kept[r]].tolist() == ref.tolist()


# ----------------------------------------------------------------------------------
# Fine top-k on given scores: exact, ties to the lower position.
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("k", [1, 7, 512, 2048])
def test_topk_exact_on_given_scores(csa2, k):
    _log(f"top-k exact: k {k}")
    wl = make_workload("topk", 3, [64 * 130, 64 * 65 + 9, 200, 64 * 70], rows_per_req=[1, 2, 1, 1], n_needles=0)
    dw = upload(wl)
    rng = np.random.default_rng(k)
    R, ld = wl.num_rows, wl.max_entries
    sc = rng.standard_normal((R, ld)).astype(np.float32)
    sc[1] = rng.integers(0, 20, size=ld).astype(np.float32)          # heavy exact ties
    sc[2, ::3] = 0.0
    sc[2, 1::3] = -0.0                                                # +0 and -0 tie
    kept_rows = []
    for r in range(R):
        b = int(wl.row_req[r])
        nb = -(-wl.n_entries(b) // 64)
        kk = np.sort(rng.choice(nb, size=min(nb, 64), replace=False))
        if nb - 1 not in kk:
            kk = np.append(kk, nb - 1)
        kept_rows.append(kk)
    kept = np.full((R, 65), -1, dtype=np.int32)
    n_kept = np.zeros(R, dtype=np.int32)
    for r, kk in enumerate(kept_rows):
        kept[r, :kk.size] = kk
        n_kept[r] = kk.size
    sel, n_sel, ss = csa2.topk(dw.rg, torch.from_numpy(sc).cuda(), torch.from_numpy(kept).cuda(),
                               torch.from_numpy(n_kept).cuda(), k=k, with_scores=True)
    sel, n_sel, ss = sel.cpu().numpy(), n_sel.cpu().numpy(), ss.cpu().numpy()
    for r in range(R):
        b = int(wl.row_req[r])
        cand = oracle.blocks_to_entries(kept_rows[r], wl.n_entries(b))
        vals = sc[r, cand].astype(np.float64)
        ref = oracle.top_k(cand, vals, k)
        assert n_sel[r] == ref.size
        assert sel[r, :n_sel[r]].tolist() == ref.tolist(), f"row {r}"
        assert np.all(sel[r, n_sel[r]:] == -1)
        assert np.array_equal(ss[r, :n_sel[r]], sc[r, ref])


@pytest.mark.parametrize("k", [7, 512])
def test_topk_exact_value_ranges(csa2, k):
    # Score ranges that the select's first pass (bins linear in the score) cannot bin
    # finely, so it must fall back to digits of the key bits, next to ones it can:
    # one huge outlier, infinities, a range of a few denormals, scores one ulp apart,
    # a heavy-tailed row with NaNs, and both signs.
    _log(f"top-k value ranges: k {k}")
    wl = make_workload("topkrange", 7, [64 * 66] * 6, rows_per_req=1, n_needles=0)
    dw = upload(wl)
    rng = np.random.default_rng(100 + k)
    R, ld = wl.num_rows, wl.max_entries
    sc = (rng.standard_normal((R, ld)) * 1e-3).astype(np.float32)
    sc[0, 17] = 1e30
    sc[1, rng.choice(ld, 40, replace=False)] = np.inf
    sc[1, rng.choice(ld, 40, replace=False)] = -np.inf
    sc[2] = rng.integers(1, 30, size=ld).astype(np.float32) * np.float32(1e-45)   # denormals
    sc[3] = np.float32(1.0) + np.arange(ld, dtype=np.float32) * np.float32(2 ** -23)   # one ulp apart
    rng.shuffle(sc[3])
    sc[4] = rng.exponential(1.0, size=ld).astype(np.float32) ** 4
    sc[4, rng.choice(ld, 100, replace=False)] = np.nan
    sc[5] = rng.standard_normal(ld).astype(np.float32) * 100
    kept_rows = []
    for r in range(R):
        nb = -(-wl.n_entries(int(wl.row_req[r])) // 64)
        kept_rows.append(np.arange(nb))
    kept = np.full((R, 66), -1, dtype=np.int32)
    n_kept = np.zeros(R, dtype=np.int32)
    for r, kk in enumerate(kept_rows):
        kept[r, :kk.size] = kk
        n_kept[r] = kk.size
    sel, n_sel, ss = csa2.topk(dw.rg, torch.from_numpy(sc).cuda(), torch.from_numpy(kept).cuda(),
                               torch.from_numpy(n_kept).cuda(), k=k, with_scores=True)
    sel, n_sel, ss = sel.cpu().numpy(), n_sel.cpu().numpy(), ss.cpu().numpy()
    for r in range(R):
        b = int(wl.row_req[r])
        cand = oracle.blocks_to_entries(kept_rows[r], wl.n_entries(b))
        ref = oracle.top_k(cand, sc[r, cand].astype(np.float64), k)
        assert n_sel[r] == ref.size, f"row {r}"
        assert sel[r, :n_sel[r]].tolist() == ref.tolist(), f"row {r}"
        assert np.array_equal(ss[r, :n_sel[r]], sc[r, ref])


def test_topk_all_entries_mode(csa2):
    _log("top-k over all entries")
    wl = make_workload("topkall", 4, [8192, 513, 512, 3], rows_per_req=1, n_needles=0)
    dw = upload(wl)
    rng = np.random.default_rng(2)
    sc = rng.integers(0, 1000, size=(wl.num_rows, wl.max_entries)).astype(np.float32)
    sel, n_sel, _ = csa2.topk(dw.rg, torch.from_numpy(sc).cuda(), k=512)
    sel, n_sel = sel.cpu().numpy(), n_sel.cpu().numpy()
    for r in range(wl.num_rows):
        n = wl.n_entries(r)
        ref = oracle.top_k(np.arange(n), sc[r, :n].astype(np.float64), 512)
        assert sel[r, :n_sel[r]].tolist() == ref.tolist()


# ----------------------------------------------------------------------------------
# Attention on a given selected set.
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("k,swa", [(512, 128), (512, 0), (100, 37), (2048, 128), (1, 1)])
def test_sparse_attn_matches_oracle(csa2, k, swa):
    _log(f"attention: k {k}, window {swa}")
    lens = [5000, 3000, 700, 64]
    wl = make_workload("attn", 31 + k + swa, lens, rows_per_req=[1, 3, 1, 1], n_needles=4,
                       swa_len=[swa, swa, 128, 0])
    dw = upload(wl)
    rng = np.random.default_rng(k)
    R = wl.num_rows
    sel = np.full((R, k), -1, dtype=np.int32)
    n_sel = np.zeros(R, dtype=np.int32)
    for r in range(R):
        n = wl.n_entries(int(wl.row_req[r]))
        m = min(k, n) if r != R - 1 else 0          # last row: window only / nothing
        s = np.sort(rng.choice(n, size=m, replace=False)) if m else np.zeros(0, dtype=np.int64)
        sel[r, :m] = s
        n_sel[r] = m
    out, lse = csa2.sparse_attn(dw.rg, dw.q, dw.main_kv, torch.from_numpy(sel).cuda(),
                                torch.from_numpy(n_sel).cuda(), dw.swa, dw.swa_scale, wl.sm_scale)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for r in range(R):
        ro, rl = oracle.joint_attention(oracle.bf16_value(wl.q[r]), oracle.row_keys(wl, r, sel[r, :n_sel[r]]),
                                        wl.sm_scale)
        rel, dl = parity.attn_error(out[r], lse[r], ro, rl)
        assert rel <= parity.ATTN_REL and dl <= parity.LSE_ABS, f"row {r}: rel {rel:.3g} lse {dl:.3g}"


@pytest.mark.parametrize("k,swa", [(2048, 128), (2048, 0), (700, 5)])
def test_sparse_attn_one_row_head_split(csa2, k, swa):
    # One row: the launch is head-split (four workgroups per split), here with up to 34
    # splits, so the merge combines many split partials per head group.
    _log(f"attention, one row (head-split): k {k}, window {swa}")
    wl = make_workload("attn1", 55 + k + swa, [9000], rows_per_req=1, n_needles=4, swa_len=[swa])
    dw = upload(wl)
    rng = np.random.default_rng(k + swa)
    n = wl.n_entries(0)
    m = min(k, n)
    sel = np.full((1, k), -1, dtype=np.int32)
    sel[0, :m] = np.sort(rng.choice(n, size=m, replace=False))
    n_sel = np.array([m], dtype=np.int32)
    out, lse = csa2.sparse_attn(dw.rg, dw.q, dw.main_kv, torch.from_numpy(sel).cuda(),
                                torch.from_numpy(n_sel).cuda(), dw.swa, dw.swa_scale, wl.sm_scale)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    ro, rl = oracle.joint_attention(oracle.bf16_value(wl.q[0]), oracle.row_keys(wl, 0, sel[0, :m]), wl.sm_scale)
    rel, dl = parity.attn_error(out[0], lse[0], ro, rl)
    assert rel <= parity.ATTN_REL and dl <= parity.LSE_ABS, f"rel {rel:.3g} lse {dl:.3g}"


def test_sparse_attn_many_rows_single_split(csa2):
    # With enough rows each row's keys go to one workgroup, which normalises and writes
    # the output itself (no split partials, no merge); some rows also span several tiles.
    R, k = 272, 200
    lens = [300 + 7 * b for b in range(R)]
    _log(f"attention: {R} rows, k {k}, one split per row")
    wl = make_workload("attnmany", 77, lens, rows_per_req=1, n_needles=0,
                       swa_len=[128 if b % 5 else b % 128 for b in range(R)])
    dw = upload(wl)
    rng = np.random.default_rng(5)
    sel = np.full((R, k), -1, dtype=np.int32)
    n_sel = np.zeros(R, dtype=np.int32)
    for r in range(R):
        n = wl.n_entries(int(wl.row_req[r]))
        m = min(k, n) - (r % 3)
        sel[r, :m] = np.sort(rng.choice(n, size=m, replace=False))
        n_sel[r] = m
    assert csa2.sparse_attn_workspace_size(dw.rg, k) == 0, "expected the single-split plan"
    out, lse = csa2.sparse_attn(dw.rg, dw.q, dw.main_kv, torch.from_numpy(sel).cuda(),
                                torch.from_numpy(n_sel).cuda(), dw.swa, dw.swa_scale, wl.sm_scale)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for r in range(0, R, 3):
        ro, rl = oracle.joint_attention(oracle.bf16_value(wl.q[r]), oracle.row_keys(wl, r, sel[r, :n_sel[r]]),
                                        wl.sm_scale)
        rel, dl = parity.attn_error(out[r], lse[r], ro, rl)
        assert rel <= parity.ATTN_REL and dl <= parity.LSE_ABS, f"row {r}: rel {rel:.3g} lse {dl:.3g}"


def test_sparse_attn_skips_invalid_positions(csa2):
    _log("attention: negative / out-of-range positions are skipped")
    wl = make_workload("attninv", 8, [1000], rows_per_req=1, n_needles=0)
    dw = upload(wl)
    sel = np.array([[5, -1, 17, 999, 5000, 3]], dtype=np.int32)
    out, lse = csa2.sparse_attn(dw.rg, dw.q, dw.main_kv, torch.from_numpy(sel).cuda(),
                                torch.tensor([6], dtype=torch.int32).cuda(), dw.swa, dw.swa_scale, wl.sm_scale)
    ro, rl = oracle.joint_attention(oracle.bf16_value(wl.q[0]), oracle.row_keys(wl, 0, np.array([5, 17, 999, 3])),
                                    wl.sm_scale)
    rel, dl = parity.attn_error(out.cpu().numpy()[0], lse.cpu().numpy()[0], ro, rl)
    assert rel <= parity.ATTN_REL and dl <= parity.LSE_ABS


def test_clock_trace_samples(csa2):
    _log("clock trace: 64 samples 2 us apart")
    n, interval = 64, 200
    out = torch.zeros(2 * n + 2, dtype=torch.int64, device="cuda")
    csa2.debug_clock_trace(out, n, interval)
    torch.cuda.synchronize()
    v = out.cpu().numpy()
    t, r = v[0:2 * n:2].astype(np.float64), v[1:2 * n:2].astype(np.float64)
    assert v[2 * n] == 0 and v[2 * n + 1] == 0, "wrote past 2n values"
    # Sample i waits until i x interval ticks after the start, so samples are at least that
    # far apart in total (one may land late and the next on time).
    assert np.all(np.diff(t) > 0) and np.all(np.diff(r) > 0) and r[-1] - r[0] >= (n - 2) * interval
    ghz = 0.1 * (t[-1] - t[0]) / (r[-1] - r[0])
    _log(f"  shader clock {ghz:.2f} GHz over {(r[-1] - r[0]) / 100:.0f} us")
    assert 0.3 < ghz < 3.0
