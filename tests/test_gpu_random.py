"""Seeded random decode workloads against the oracle (needs an MI355X): request lengths
from empty to 140K entries, 1-16 rows per request, window lengths 0-128, k and n_keep
across their range, both Q/P routes, contiguous and paged pools, and the candidate-only
scan mode checked against the full scan."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
from synth import make_workload, to_paged
from synth.device import upload

pytestmark = pytest.mark.gpu

CASES = 16


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


def draw_case(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 10))
    lens = []
    for _ in range(B):
        kind = int(rng.integers(0, 6))
        if kind == 0:
            n = rng.integers(0, 200)
        elif kind == 1:
            n = 64 * rng.integers(1, 300) + rng.integers(-1, 2)
        elif kind == 2:
            n = rng.integers(1000, 20000)
        elif kind == 3:
            n = rng.integers(20000, 45000)
        elif kind == 4:
            n = rng.integers(200, 1000)
        else:
            n = rng.integers(60000, 140000) if rng.random() < 0.5 else rng.integers(45000, 60000)
        lens.append(max(0, int(n)))
    return dict(
        lens=lens,
        rows=[int(rng.choice([1, 1, 1, 2, 3, 6, 16])) for _ in range(B)],
        swa=[int(rng.choice([0, 1, 5, 77, 128, 128])) for _ in range(B)],
        k=int(rng.choice([1, 7, 100, 300, 512, 512, 2048])),
        n_keep=int(rng.choice([1, 4, 20, 64, 64, 128])),
        newest=bool(rng.integers(0, 2)),
        mx=bool(rng.random() < 1 / 3),
        paged=bool(rng.integers(0, 2)),
        scan_mode=int(rng.integers(0, 2)),
        needles=int(rng.choice([0, 4, 16])),
    )


def run(csa2, wl, c, scan_mode):
    dw = upload(wl)
    d = csa2.Decoder(*dw.decode_inputs(), k=c["k"], n_keep=c["n_keep"], keep_newest=c["newest"],
                     sm_scale=wl.sm_scale, qp_route=csa2.QP_MXFP8 if c["mx"] else csa2.QP_BF16,
                     scan_mode=scan_mode)
    d.run()
    torch.cuda.synchronize()
    return {x: getattr(d, y).cpu().numpy() for x, y in
            (("out", "out"), ("lse", "lse"), ("sel", "sel_idx"), ("n_sel", "n_sel"), ("kept", "kept"),
             ("n_kept", "n_kept"))}


def mx_attention_ok(wl, got, r):
    """The MXFP8 route's attention within the oracle's bound for two P roundings."""
    sel = got["sel"][r, :got["n_sel"][r]]
    codes, scales = oracle.row_key_codes(wl, r, sel)
    ro, rl, bound = oracle.joint_attention_mx(oracle.bf16_value(wl.q[r]), codes, scales, wl.sm_scale,
                                              with_bound=True)
    err = np.abs(got["out"][r].astype(np.float64) - ro)
    both = np.isneginf(got["lse"][r]) & np.isneginf(rl)
    dl = np.where(both, 0.0, np.abs(got["lse"][r] - rl))
    return bool(np.all(err <= bound * (1 + 1e-4) + 1e-7) and dl.max() <= 2e-3)


@pytest.mark.parametrize("case", range(CASES))
def test_random_decode_matches_oracle(csa2, case):
    seed = 7000 + case
    c = draw_case(seed)
    _log(f"case {case} (seed {seed}): lens {c['lens']} rows {c['rows']} swa {c['swa']} k {c['k']} "
         f"n_keep {c['n_keep']} newest {int(c['newest'])} mx {int(c['mx'])} paged {int(c['paged'])} "
         f"scan_mode {c['scan_mode']}")
    wl = make_workload(f"random{case}", seed, c["lens"], rows_per_req=c["rows"], n_needles=c["needles"],
                       swa_len=c["swa"])
    wlr = to_paged(wl, seed=seed) if c["paged"] else wl
    got = run(csa2, wlr, c, c["scan_mode"])
    if c["scan_mode"]:
        # The candidate-only scan scores only the kept blocks: the same selection and output.
        full = run(csa2, wlr, c, 0)
        for key in got:
            assert np.array_equal(got[key], full[key]), key
    refs = oracle.decode(wl, k=c["k"], n_keep=c["n_keep"], keep_newest=int(c["newest"]))
    for r, ref in enumerate(refs):
        rep = parity.check_row(wl, r, ref, got["kept"][r, :got["n_kept"][r]], got["sel"][r, :got["n_sel"][r]],
                               got["out"][r], got["lse"][r], k=c["k"], n_keep=c["n_keep"])
        if c["mx"]:
            # Kept blocks and the selected set as usual; attention against the route's bound.
            assert all(m.startswith("attention") for m in rep["msgs"]), (r, rep["msgs"][:2])
            assert mx_attention_ok(wl, got, r), r
        else:
            assert rep["ok"], (r, rep["msgs"][:2])
