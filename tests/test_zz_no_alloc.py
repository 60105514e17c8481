"""csa2_decode_static, the decode entry point that allocates nothing (its workspace is
the library's static per-device buffer), against csa2_decode on the same inputs."""
import ctypes
import os
import sys

import numpy as np
import pytest
import torch

import sparse_decode_attention_csa2_amd as csa2
from synth import make_config
from synth.device import upload


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(csa2.LIB_PATH):
        pytest.fail("libcsa2.so is not built (run __graft_entry__.build())")
    return csa2.load_library()


def test_static_decode_rejects_workspaces_beyond_the_limit(lib):
    # 64 rows of 2^24 entries need a 4 GiB score buffer: rejected on the host, nothing
    # launched (no device memory is touched, so this runs without a GPU).
    a = csa2._DecodeArgs()
    rg = a.rg
    rg.num_requests, rg.num_rows = 64, 64
    for f in ("entry_off", "block_off", "row_off", "row_req", "row_swa_start", "row_swa_len"):
        setattr(rg, f, 0x10000)
    rg.max_entries = rg.total_entries = 1 << 24
    rg.total_blocks, rg.swa_tokens, rg.max_rows_per_request = 1 << 18, 128, 1
    a.k, a.n_keep, a.keep_newest = 512, 64, 1
    need = lib.csa2_decode_workspace_size(ctypes.byref(a))
    assert need > csa2.STATIC_WS_BYTES
    assert lib.csa2_decode_static(ctypes.byref(a), None) == csa2.ERR_WORKSPACE_TOO_SMALL
    assert b"static workspace" in lib.csa2_last_error()
    assert lib.csa2_decode_static(None, None) == csa2.ERR_INVALID_ARG


def _outputs(d, wl):
    torch.cuda.synchronize()
    got = {k: getattr(d, k).cpu().numpy().copy() for k in ("out", "lse", "sel_idx", "n_sel", "kept", "n_kept")}
    sc = d.scores.cpu().numpy()
    got["scores"] = np.concatenate([sc[r, :wl.n_entries(int(wl.row_req[r]))] for r in range(wl.num_rows)])
    return got


def _poison(d):
    for t in (d.out, d.lse, d.scores):
        t.fill_(float("nan"))
    for t in (d.sel_idx, d.n_sel, d.kept, d.n_kept):
        t.fill_(-7)


@pytest.mark.gpu
def test_static_decode_matches_decode_twice_then_smaller(lib):
    # Two static calls in a row, the second on a smaller batch (the buffer then still
    # holds the first call's contents); each is compared bit for bit with csa2_decode on
    # the same inputs, with the outputs poisoned before every call; both Q/P routes (the
    # MXFP8 route's workspace also holds the rounded query).
    for route, cfg in ((csa2.QP_BF16, 3), (csa2.QP_BF16, 0), (csa2.QP_MXFP8, 3), (csa2.QP_MXFP8, 0)):
        wl = make_config(cfg)
        dw = upload(wl)
        d = csa2.Decoder(*dw.decode_inputs(), k=wl.k, n_keep=wl.n_keep, sm_scale=wl.sm_scale, qp_route=route)
        _log(f"static decode, {wl.name}, route {route}: {wl.num_rows} rows, workspace {d.ws_bytes} bytes "
             f"(static buffer {csa2.STATIC_WS_BYTES})")
        assert d.ws_bytes <= csa2.STATIC_WS_BYTES
        _poison(d)
        d.run_static()
        st = _outputs(d, wl)
        _poison(d)
        d.run()
        ref = _outputs(d, wl)
        for key in ref:
            a, b = st[key], ref[key]
            if a.dtype == np.float32:
                a, b = a.view(np.uint32), b.view(np.uint32)
            assert np.array_equal(a, b), f"{wl.name}: {key}"
        assert np.isfinite(st["out"]).all()
        del d, dw
        torch.cuda.empty_cache()
