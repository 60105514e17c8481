"""Paged pools, per-row visible lengths and the score check on the HIP path, against
the contiguous path (bit-exact: the same arithmetic on the same values) and against the
oracle (needs an MI355X)."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
from synth import make_config, make_workload, to_paged, verify_row_len
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


def run_decode(csa2, wl, k=None, n_keep=None, scan_mode=0):
    dw = upload(wl)
    d = csa2.Decoder(*dw.decode_inputs(), k=wl.k if k is None else k, n_keep=wl.n_keep if n_keep is None else n_keep,
                     keep_newest=bool(wl.keep_newest), sm_scale=wl.sm_scale, scan_mode=scan_mode)
    d.run()
    torch.cuda.synchronize()
    return dict(out=d.out.cpu().numpy(), lse=d.lse.cpu().numpy(), sel=d.sel_idx.cpu().numpy(),
                n_sel=d.n_sel.cpu().numpy(), kept=d.kept.cpu().numpy(), n_kept=d.n_kept.cpu().numpy(),
                scores=d.scores.cpu().numpy())


def same(a, b):
    """Bit-for-bit equality (NaN where both are NaN)."""
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype.kind == "f":
        a32, b32 = a.astype(np.float32), b.astype(np.float32)
        nan = np.isnan(a32) & np.isnan(b32)
        return bool(np.all(nan | (a32.view(np.uint32) == b32.view(np.uint32))))
    return bool(np.array_equal(a, b))


def judge(wl, got, k=None, n_keep=None, rows=None):
    rows = list(range(wl.num_rows)) if rows is None else rows
    refs = oracle.decode(wl, rows=rows, k=k, n_keep=n_keep)
    bad = []
    for r, ref in zip(rows, refs):
        rep = parity.check_row(wl, r, ref, got["kept"][r, :got["n_kept"][r]], got["sel"][r, :got["n_sel"][r]],
                               got["out"][r], got["lse"][r], k=k, n_keep=n_keep)
        if not rep["ok"]:
            bad.append(rep)
    _log(f"  {len(rows)} rows judged, {len(bad)} bad")
    assert not bad, "; ".join(f"row {rp['row']}: {' | '.join(rp['msgs'])}" for rp in bad[:5])


def edge_workload(seed=41):
    lens = [0, 1, 63, 64, 65, 511, 513, 64 * 64, 64 * 64 + 1, 64 * 65 + 63, 20000]
    swa = [0, 1, 128, 5, 0, 128, 77, 128, 128, 128, 128]
    rows = [1, 1, 2, 1, 1, 3, 1, 1, 6, 1, 2]
    return make_workload("edge", seed, lens, rows_per_req=rows, n_needles=4, swa_len=swa)


@pytest.mark.parametrize("cfg,scan_mode", [(0, 0), (2, 0), (3, 0), (3, 1), (1, 0)])
def test_paged_decode_equals_contiguous(csa2, cfg, scan_mode):
    wl = make_config(cfg)
    pw = to_paged(wl)
    _log(f"config {cfg} paged ({pw.total_pages} pages, scan mode {scan_mode})")
    a = run_decode(csa2, wl, scan_mode=scan_mode)
    b = run_decode(csa2, pw, scan_mode=scan_mode)
    for key in ("sel", "n_sel", "kept", "n_kept", "out", "lse", "scores"):
        assert same(a[key], b[key]), key


def test_paged_decode_edge_matches_oracle(csa2):
    pw = to_paged(edge_workload())
    _log(f"edge workload paged: {pw.num_rows} rows")
    for scan_mode in (0, 1):
        judge(pw, run_decode(csa2, pw, scan_mode=scan_mode))


def test_verify_row_len_matches_oracle(csa2):
    wl = make_config(3)
    wl.row_len = verify_row_len(wl)
    _log(f"verify_8x6 with row lengths {wl.row_len[:6].tolist()} ...")
    got = run_decode(csa2, wl)
    judge(wl, got, rows=list(range(0, wl.num_rows, 5)))
    for r in range(wl.num_rows):
        assert got["n_sel"][r] == 0 or got["sel"][r, :got["n_sel"][r]].max() < wl.row_len[r]
    # Candidate-only scan and paged pools give the same bits.
    assert same(run_decode(csa2, wl, scan_mode=1)["out"], got["out"])
    pw = to_paged(wl)
    pg = run_decode(csa2, pw)
    for key in ("sel", "n_sel", "kept", "n_kept", "out", "lse"):
        assert same(pg[key], got[key]), key


def test_random_row_len_matches_oracle(csa2):
    wl = edge_workload(43)
    rng = np.random.default_rng(7)
    rl = np.zeros(wl.num_rows, dtype=np.int64)
    for r in range(wl.num_rows):
        n = wl.n_entries(int(wl.row_req[r]))
        rl[r] = [0, n, int(rng.integers(0, n + 1)), n + 100, (n // 64) * 64][r % 5]
    wl.row_len = rl
    _log(f"edge workload with row lengths {rl.tolist()}")
    for scan_mode in (0, 1):
        got = run_decode(csa2, wl, k=300, n_keep=20, scan_mode=scan_mode)
        judge(wl, got, k=300, n_keep=20)
        for r in range(wl.num_rows):
            if rl[r] == 0:
                assert got["n_sel"][r] == 0 and got["n_kept"][r] == 0
    judge(to_paged(wl), run_decode(csa2, to_paged(wl), k=300, n_keep=20), k=300, n_keep=20)


def test_nan_scores_are_never_selected(csa2):
    wl = make_workload("nan", 33, [64 * 80 + 9, 3000], rows_per_req=[2, 1], n_needles=16)
    for b in range(2):
        wl.idx_k[int(wl.entry_off[b]) + wl.needles[b], 64] = 255     # NaN scale: NaN score
    wl.blk_sum[[3, 80]] = 0x7FC0                                     # NaN summaries (80 = newest of request 0)
    _log("NaN-scored entries and blocks")
    for scan_mode in (0, 1):
        got = run_decode(csa2, wl, k=200, n_keep=20, scan_mode=scan_mode)
        judge(wl, got, k=200, n_keep=20)
        for r in range(wl.num_rows):
            b = int(wl.row_req[r])
            sel = set(got["sel"][r, :got["n_sel"][r]].tolist())
            assert not sel & set(wl.needles[b].tolist())
        assert 3 not in got["kept"][0, :got["n_kept"][0]] and 80 in got["kept"][0, :got["n_kept"][0]]


def test_standalone_entry_points_paged_equal_contiguous(csa2):
    wl = edge_workload(45)
    wl.row_len = verify_row_len(wl)
    pw = to_paged(wl)
    da, dp = upload(wl), upload(pw)
    _log("index_score / block_filter / topk / sparse_attn, paged vs contiguous")
    sa = csa2.index_score(da.rg, da.idx_k, da.q_idx, da.w)
    sp = csa2.index_score(dp.rg, dp.idx_k, dp.q_idx, dp.w)
    assert same(sa.cpu().numpy(), sp.cpu().numpy())
    ka, nka, bsa = csa2.block_filter(da.rg, da.blk_sum, da.q_idx, da.w, n_keep=16)
    kp, nkp, bsp = csa2.block_filter(dp.rg, dp.blk_sum, dp.q_idx, dp.w, n_keep=16)
    assert same(ka.cpu().numpy(), kp.cpu().numpy()) and same(nka.cpu().numpy(), nkp.cpu().numpy())
    assert same(bsa.cpu().numpy(), bsp.cpu().numpy())
    ska = csa2.index_score(da.rg, da.idx_k, da.q_idx, da.w, kept=ka, n_kept=nka)
    skp = csa2.index_score(dp.rg, dp.idx_k, dp.q_idx, dp.w, kept=kp, n_kept=nkp)
    assert same(ska.cpu().numpy(), skp.cpu().numpy())
    sel_a, ns_a, _ = csa2.topk(da.rg, sa, ka, nka, k=100)
    sel_p, ns_p, _ = csa2.topk(dp.rg, sp, kp, nkp, k=100)
    assert same(sel_a.cpu().numpy(), sel_p.cpu().numpy()) and same(ns_a.cpu().numpy(), ns_p.cpu().numpy())
    # Attention with positions the rows do not see mixed in: they carry no key.
    sel_x = sel_a.clone()
    sel_x[:, -1] = 10 ** 6
    ns_x = torch.full_like(ns_a, sel_x.shape[1])
    oa, la = csa2.sparse_attn(da.rg, da.q, da.main_kv, sel_x, ns_x, da.swa, da.swa_scale)
    op, lp = csa2.sparse_attn(dp.rg, dp.q, dp.main_kv, sel_x, ns_x, dp.swa, dp.swa_scale)
    torch.cuda.synchronize()
    assert same(oa.cpu().numpy(), op.cpu().numpy()) and same(la.cpu().numpy(), lp.cpu().numpy())
    sel_np = sel_x.cpu().numpy()
    for r in range(0, wl.num_rows, 3):
        ro, rl = oracle.joint_attention(oracle.bf16_value(wl.q[r]), oracle.row_keys(wl, r, sel_np[r]), wl.sm_scale)
        rel, dl = parity.attn_error(oa[r].cpu().numpy(), la[r].cpu().numpy(), ro, rl)
        assert rel <= parity.ATTN_REL and dl <= parity.LSE_ABS, (r, rel, dl)


def test_out_of_range_page_ids_are_clamped(csa2):
    # Page ids outside 0 .. total_pages-1 address the nearest valid page (the documented
    # clamp): the result equals a decode whose page table holds the clamped ids.  Whole
    # pages and no spare pages, so every page holds real records (no random bytes).
    pw = to_paged(make_workload("clamp", 47, [64 * 30, 64 * 14], rows_per_req=[2, 1], n_needles=4),
                  spare_pages=0)
    bad = pw.page_table.copy()
    bad[0, 3] = -5
    bad[1, 2] = pw.total_pages + 100
    clamped = np.clip(bad, 0, pw.total_pages - 1)
    pw.page_table = bad
    got = run_decode(csa2, pw, k=200, n_keep=16)
    pw.page_table = clamped
    ref = run_decode(csa2, pw, k=200, n_keep=16)
    for key in ("sel", "kept", "out", "lse"):
        assert same(got[key], ref[key]), key
    judge(pw, got, k=200, n_keep=16)


def test_sixteen_rows_per_request_long(csa2):
    # The 8-pair scan (16 rows share one key stream) over a request of 40,000+ entries
    # (many chunks per wave and a ragged tail), contiguous and paged, both scan modes.
    wl = make_workload("rows16long", 49, [64 * 640 + 21, 3000], rows_per_req=[16, 2], n_needles=12)
    _log("16 rows per request, 40,981 entries")
    for w in (wl, to_paged(wl)):
        refs = oracle.decode(w)
        for scan_mode in (0, 1):
            got = run_decode(csa2, w, scan_mode=scan_mode)
            bad = []
            for r, ref in enumerate(refs):
                rep = parity.check_row(w, r, ref, got["kept"][r, :got["n_kept"][r]], got["sel"][r, :got["n_sel"][r]],
                                       got["out"][r], got["lse"][r])
                if not rep["ok"]:
                    bad.append(rep)
            _log(f"  paged {w.page_table is not None}, scan mode {scan_mode}: {len(refs)} rows, {len(bad)} bad")
            assert not bad, "; ".join(f"row {rp['row']}: {' | '.join(rp['msgs'])}" for rp in bad[:5])


def test_sixteen_rows_per_request_paged_with_row_len(csa2):
    # The largest row group (16 rows share one key stream: the 8-pair scan), paged, with
    # every row seeing a different prefix, in both scan modes.
    wl = make_workload("rows16", 48, [64 * 70 + 33, 5000], rows_per_req=[16, 3], n_needles=8)
    rl = np.array([64 * 70 + 33 - 37 * j for j in range(16)] + [5000, 64, 4999], dtype=np.int64)
    wl.row_len = rl
    pw = to_paged(wl)
    _log("16 rows per request, paged, row lengths")
    for scan_mode in (0, 1):
        got = run_decode(csa2, pw, k=256, n_keep=24, scan_mode=scan_mode)
        judge(pw, got, k=256, n_keep=24)
