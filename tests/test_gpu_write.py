"""csa2_cache_write against the oracle (needs an MI355X): the records it writes, bit for
bit except where the fp32 pipeline and the oracle's fp64 one fall on opposite sides of a
rounding tie; the block summaries recomputed from the records it wrote; the ring slots;
untouched rows left alone; contiguous and paged pools."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import make_config, make_workload, make_write_inputs, to_paged
from synth.device import upload

pytestmark = pytest.mark.gpu

E2M1_TIES = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


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


def _dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def run_write(csa2, wl, w, eps=1e-6):
    dw = upload(wl)
    ring_kv, ring_idx = _dev(w["ring_kv"]), _dev(w["ring_idx"])
    csa2.cache_write(dw.rg, _dev(w["row_pos"]), _dev(w["kv_tok"]), _dev(w["idx_tok"]), ring_kv, ring_idx,
                     _dev(w["gamma_kv"]), _dev(w["gamma_idx"]), dw.main_kv, dw.idx_k, dw.blk_sum, eps)
    torch.cuda.synchronize()
    u16 = lambda t: t.cpu().numpy().view(np.uint16)
    return dict(main_kv=dw.main_kv.cpu().numpy(), idx_k=dw.idx_k.cpu().numpy(), blk_sum=u16(dw.blk_sum),
                ring_kv=u16(ring_kv), ring_idx=u16(ring_idx))


def _allowed(y, block, rel=1e-5):
    """Elements whose code may differ: |y| / 2^e within rel of an E2M1 tie, or the whole
    block when its maximum is within rel of a power of two (the scale decision)."""
    y = np.asarray(y, dtype=np.float64).reshape(-1, block)
    amax = np.abs(y).max(axis=1, keepdims=True)
    _, fe = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.clip(fe - 1 - 2, -127, 127)
    v = np.abs(y) / np.ldexp(1.0, e)
    near_tie = (np.abs(v[..., None] - E2M1_TIES) <= rel * E2M1_TIES).any(axis=-1)
    frac = amax / np.ldexp(1.0, fe - 1)                       # in [1, 2)
    near_pow2 = (frac - 1.0 <= rel) | (2.0 - frac <= rel)
    return (near_tie | near_pow2).reshape(-1), near_pow2[:, 0]


def check_write(wl, got, ref):
    rows_written = []
    n_diff = 0
    for (b, t), (yk, yi) in ref["written"].items():
        row = int(oracle.entry_rows(wl, b, np.array([t]))[0])
        rows_written.append(row)
        for pool, y, block, dim in (("main_kv", yk, 16, 512), ("idx_k", yi, 32, 128)):
            g, r = got[pool][row], ref[pool][row]
            if np.array_equal(g, r):
                continue
            el_ok, blk_ok = _allowed(y, block)
            gc = np.stack([g[:dim // 2] & 15, g[:dim // 2] >> 4], axis=1).reshape(-1)
            rc = np.stack([r[:dim // 2] & 15, r[:dim // 2] >> 4], axis=1).reshape(-1)
            bad = (gc != rc) & ~el_ok
            bad_scale = (g[dim // 2:] != r[dim // 2:]) & ~blk_ok
            assert not bad.any() and not bad_scale.any(), (pool, b, t, np.flatnonzero(bad)[:8])
            n_diff += int((gc != rc).sum())
    # Nothing else in the pools moved.
    keep = np.ones(wl.idx_k.shape[0], dtype=bool)
    keep[rows_written] = False
    assert np.array_equal(got["idx_k"][keep], wl.idx_k[keep]) and np.array_equal(got["main_kv"][keep], wl.main_kv[keep])
    # Summaries: recomputed from the records the kernel wrote; all others untouched.
    touched = set()
    for (b, t) in ref["written"]:
        touched.add((b, t // 64))
    srows = []
    for b, j in sorted(touched):
        n = wl.n_entries(b)
        cnt = min(64, n - 64 * j)
        keys = oracle.dequant_idx(got["idx_k"][oracle.entry_rows(wl, b, np.arange(64 * j, 64 * j + cnt))])
        srow = int(oracle.block_rows(wl, b, j + 1)[j])
        srows.append(srow)
        assert np.array_equal(got["blk_sum"][srow], oracle.bf16_rne(keys.mean(axis=0))), (b, j)
    skeep = np.ones(wl.blk_sum.shape[0], dtype=bool)
    skeep[srows] = False
    assert np.array_equal(got["blk_sum"][skeep], wl.blk_sum[skeep])
    assert np.array_equal(got["ring_kv"], ref["ring_kv"]) and np.array_equal(got["ring_idx"], ref["ring_idx"])
    _log(f"  {len(ref['written'])} entries written, {n_diff} codes at rounding ties differ, "
         f"{len(touched)} summaries")


@pytest.mark.parametrize("last_even", [True, False])
def test_cache_write_verify_rows(csa2, last_even):
    wl = make_config(3)          # 8 requests x 6 verify rows over 16,384 entries each
    w = make_write_inputs(wl, 61, last_even)
    _log(f"verify_8x6 cache write, last position {'even' if last_even else 'odd'}")
    got = run_write(csa2, wl, w)
    ref = oracle.cache_write(wl, w["row_pos"], w["kv_tok"], w["idx_tok"], w["ring_kv"], w["ring_idx"],
                             w["gamma_kv"], w["gamma_idx"])
    check_write(wl, got, ref)


def test_cache_write_ragged_and_paged(csa2):
    # Requests of 1, 63, 64, 65 and 200 entries (new entries straddle block edges), 1 to
    # 16 rows each, contiguous and paged.
    wl = make_workload("wr", 62, [1, 63, 64, 65, 200, 130], rows_per_req=[1, 2, 3, 4, 16, 5], n_needles=2)
    for paged in (False, True):
        ww = to_paged(wl) if paged else wl
        w = make_write_inputs(ww, 63)
        _log(f"ragged cache write, paged={paged}")
        got = run_write(csa2, ww, w)
        ref = oracle.cache_write(ww, w["row_pos"], w["kv_tok"], w["idx_tok"], w["ring_kv"], w["ring_idx"],
                                 w["gamma_kv"], w["gamma_idx"])
        check_write(ww, got, ref)


@pytest.mark.parametrize("case", range(8))
def test_cache_write_random_shapes(csa2, case):
    # Seeded random requests: lengths from 1 entry to a few blocks (block edges included),
    # 1 to 16 rows each, the last position even or odd, contiguous or paged pools.
    rng = np.random.default_rng(900 + case)
    B = int(rng.integers(1, 9))
    lens = [int(rng.choice([rng.integers(1, 70), 64 * rng.integers(1, 40) + rng.integers(-1, 2),
                            rng.integers(70, 5000)])) for _ in range(B)]
    lens = [max(1, n) for n in lens]
    rows = [min(int(rng.integers(1, 17)), 2 * n - 1) for n in lens]   # positions stay >= 0
    wl = make_workload(f"wrand{case}", 910 + case, lens, rows_per_req=rows, n_needles=0)
    ww = to_paged(wl, seed=920 + case) if rng.integers(0, 2) else wl
    w = make_write_inputs(ww, 930 + case, last_even=bool(rng.integers(0, 2)))
    _log(f"random cache write {case}: lens {lens} rows {rows} paged {ww is not wl}")
    got = run_write(csa2, ww, w)
    ref = oracle.cache_write(ww, w["row_pos"], w["kv_tok"], w["idx_tok"], w["ring_kv"], w["ring_idx"],
                             w["gamma_kv"], w["gamma_idx"])
    check_write(ww, got, ref)


def test_written_cache_decodes_like_the_oracle(csa2):
    # Write the last entries of a verify batch, then decode over the written pools.
    from oracle import parity
    wl = make_workload("wd", 64, [3000, 5000], rows_per_req=[6, 6], n_needles=4)
    w = make_write_inputs(wl, 65)
    got = run_write(csa2, wl, w)
    wl.main_kv, wl.idx_k, wl.blk_sum = got["main_kv"], got["idx_k"], got["blk_sum"]
    dw = upload(wl)
    d = csa2.decode(*dw.decode_inputs(), k=256, n_keep=16, sm_scale=wl.sm_scale)
    torch.cuda.synchronize()
    refs = oracle.decode(wl, k=256, n_keep=16)
    for r in range(wl.num_rows):
        rep = parity.check_row(wl, r, refs[r], d.kept.cpu().numpy()[r, :d.n_kept.cpu()[r]],
                               d.sel_idx.cpu().numpy()[r, :d.n_sel.cpu()[r]], d.out.cpu().numpy()[r],
                               d.lse.cpu().numpy()[r], k=256, n_keep=16)
        assert rep["ok"], rep["msgs"]
