"""The MXFP8 Q/P route of the attention (needs an MI355X): the kernels' MXFP8 rounding
bit for bit against the oracle, and csa2_decode with CSA2_QP_MXFP8 against the oracle's
route within the rounding bound the oracle derives (the implementation rounds P against
the running maximum of its own key range, the oracle against the row's maximum, so
their P roundings are two independent roundings of the same weights)."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import make_config, make_workload, to_paged
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


def run_decode(csa2, wl, route, k=None, n_keep=None):
    dw = upload(wl)
    d = csa2.Decoder(*dw.decode_inputs(), k=wl.k if k is None else k, n_keep=wl.n_keep if n_keep is None else n_keep,
                     keep_newest=bool(wl.keep_newest), sm_scale=wl.sm_scale, qp_route=route)
    d.run()
    torch.cuda.synchronize()
    return dict(out=d.out.cpu().numpy(), lse=d.lse.cpu().numpy(), sel=d.sel_idx.cpu().numpy(),
                n_sel=d.n_sel.cpu().numpy(), kept=d.kept.cpu().numpy(), n_kept=d.n_kept.cpu().numpy())


def judge_mx(wl, got, rows=None):
    """Every (head, dim) within the oracle's bound for two independent P roundings (plus
    1e-4 of it for fp32 arithmetic); lse (unrounded p, identical rounded Q) within 2e-3."""
    rows = range(wl.num_rows) if rows is None else rows
    worst = 0.0
    for r in rows:
        sel = got["sel"][r, :got["n_sel"][r]]
        codes, scales = oracle.row_key_codes(wl, r, sel)
        ro, rl, bound = oracle.joint_attention_mx(oracle.bf16_value(wl.q[r]), codes, scales, wl.sm_scale,
                                                  with_bound=True)
        err = np.abs(got["out"][r].astype(np.float64) - ro)
        tol = bound * (1 + 1e-4) + 1e-7
        assert np.all(err <= tol), (r, float((err - tol).max()))
        both_inf = np.isneginf(got["lse"][r]) & np.isneginf(rl)
        dl = np.where(both_inf, 0.0, np.abs(got["lse"][r] - rl))
        assert dl.max() <= 2e-3, (r, float(dl.max()))
        worst = max(worst, float((err / np.maximum(tol, 1e-30)).max()))
    _log(f"  worst error / bound {worst:.3f}")


def test_mxfp8_rounding_matches_oracle(csa2):
    rng = np.random.default_rng(21)
    blocks = []
    for mag in (1e-30, 1e-6, 2.0 ** -20, 0.1, 1.0, 3.7, 448.0, 1e5, 2.0 ** 100):
        for _ in range(64):
            blocks.append(rng.standard_normal(32) * mag)
    # Every E4M3 grid point and every midpoint between neighbours (ties), at scale 2^0:
    # a block maximum of 448 keeps the shared exponent at 0.
    grid = oracle.E4M3_GRID
    mids = (grid[:-1] + grid[1:]) / 2
    vals = np.concatenate([grid, mids, -mids, grid * 1.0001, mids * 0.9999, [470.0, 500.0, 511.0]])
    for i in range(0, vals.size, 31):
        blocks.append(np.concatenate([[448.0], vals[i:i + 31], np.zeros(max(0, 31 - vals[i:i + 31].size))]))
    z = rng.standard_normal(32)
    z[[1, 5]] = [0.0, z.max() * 1e-5]
    blocks += [z, np.zeros(32)]
    x = np.stack(blocks).astype(np.float32)
    # The same blocks rounded to bf16 (the query's type) take the bf16-input rounding:
    # every grid point and midpoint above is a bf16 value already; add the random blocks
    # as bf16 and a block of bf16 subnormals (shared exponent at its floor of -127; the
    # results are multiples of 2^-133, so bf16 holds them).
    xb = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    sub = (rng.integers(1, 128, 32) * rng.choice([-1.0, 1.0], 32) * 2.0 ** -133).astype(np.float32)
    x = np.concatenate([x, xb, sub[None]])
    exact = (x.view(np.uint32) & 0xFFFF) == 0
    assert exact[-1].all() and exact.all(axis=1).sum() >= x.shape[0] // 2
    got = csa2.debug_mxfp8(torch.from_numpy(x.reshape(-1)).cuda()).cpu().numpy().reshape(x.shape)
    ref = oracle.mxfp8_round(x.astype(np.float64))
    _log(f"mxfp8 rounding: {x.shape[0]} blocks")
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("cfg", [0, 3])
def test_mx_route_decode_matches_oracle(csa2, cfg):
    wl = make_config(cfg)
    _log(f"config {cfg} ({wl.name}) MXFP8 route")
    got = run_decode(csa2, wl, csa2.QP_MXFP8)
    ref = run_decode(csa2, wl, csa2.QP_BF16)
    # The route changes only the attention arithmetic.
    for key in ("sel", "n_sel", "kept", "n_kept"):
        assert np.array_equal(got[key], ref[key]), key
    assert not np.array_equal(got["out"], ref["out"])
    judge_mx(wl, got, rows=range(0, wl.num_rows, 5))


@pytest.mark.parametrize("cfg, rows", [(1, None), (5, [0, 21, 42, 63])])
def test_mx_route_full_size_matches_oracle(csa2, cfg, rows):
    # The MXFP8 route at the sizes bench.py times it (one 128K row; sampled rows of the
    # 64 x 128K batch): same selections as the BF16 route, attention within the oracle's
    # bound for the route.
    wl = make_config(cfg)
    _log(f"config {cfg} ({wl.name}) MXFP8 route, full size")
    got = run_decode(csa2, wl, csa2.QP_MXFP8)
    ref = run_decode(csa2, wl, csa2.QP_BF16)
    for key in ("sel", "n_sel", "kept", "n_kept"):
        assert np.array_equal(got[key], ref[key]), key
    judge_mx(wl, got, rows=rows)


def test_mx_route_edge_and_paged(csa2):
    lens = [0, 1, 63, 64, 65, 511, 513, 64 * 65 + 63, 20000]
    swa = [0, 1, 128, 5, 0, 128, 77, 128, 128]
    rows = [1, 1, 2, 1, 1, 3, 1, 1, 2]
    wl = make_workload("edge", 51, lens, rows_per_req=rows, n_needles=4, swa_len=swa)
    _log(f"edge workload MXFP8 route: {wl.num_rows} rows")
    got = run_decode(csa2, wl, csa2.QP_MXFP8, k=300, n_keep=20)
    judge_mx(wl, got)
    pg = run_decode(csa2, to_paged(wl), csa2.QP_MXFP8, k=300, n_keep=20)
    assert np.array_equal(pg["out"], got["out"]) and np.array_equal(pg["lse"], got["lse"])


def test_mx_route_single_tile_rounds_like_the_oracle(csa2):
    # 32 selected entries + 16 window tokens = one 64-key tile in one workgroup, whose
    # running maximum is the row's maximum: both sides round the same weights, so they
    # differ only where fp32 and fp64 weights straddle a rounding midpoint (a step of at
    # most 1/8 of that weight).  Allow four such steps per head instead of the full bound.
    wl = make_workload("one_tile", 52, [3000], rows_per_req=1, n_needles=4, swa_len=16)
    got = run_decode(csa2, wl, csa2.QP_MXFP8, k=32, n_keep=8)
    r = 0
    sel = got["sel"][r, :got["n_sel"][r]]
    assert sel.size == 32
    codes, scales = oracle.row_key_codes(wl, r, sel)
    q = oracle.bf16_value(wl.q[r])
    ro, rl = oracle.joint_attention_mx(q, codes, scales, wl.sm_scale)
    z = (oracle.mxfp8_round(q) @ codes.T) * scales[None, :] * wl.sm_scale
    p = np.exp(z - z.max(axis=1, keepdims=True))
    w = p * scales[None, :]
    step = (2.0 ** -3) * np.abs(w)[:, :, None] * np.abs(codes)[None, :, :] / p.sum(axis=1)[:, None, None]
    tol = 4 * step.max(axis=1) + 1e-6 * np.abs(ro) + 1e-7
    err = np.abs(got["out"][r] - ro)
    _log(f"  single tile: max error {err.max():.3g}, max error / tolerance {(err / tol).max():.3f}")
    assert np.all(err <= tol)
