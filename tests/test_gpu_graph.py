"""Graph replay of the decode chain equals eager execution, replay after replay, and
decoders on concurrent streams equal their lone runs (needs an MI355X)."""
import os

import numpy as np
import pytest
import torch

from synth import make_config, make_workload
from synth.device import upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    import sparse_decode_attention_csa2_amd as m
    if not os.path.exists(m.LIB_PATH):
        pytest.fail("libcsa2.so missing: the HIP path must be built before GPU tests")
    m.load_library()
    return m


def _snap(d):
    return [t.clone() for t in (d.out, d.lse, d.sel_idx, d.n_sel, d.kept, d.n_kept)]


def test_graph_replay_matches_eager(csa2):
    wl = make_config(3)
    other = make_workload("other", 5, [5000, 300], rows_per_req=[2, 1])
    dw, ow = upload(wl), upload(other)
    d = csa2.Decoder(*dw.decode_inputs(), sm_scale=wl.sm_scale)
    o = csa2.Decoder(*ow.decode_inputs(), sm_scale=other.sm_scale)
    d.run()
    o.run()
    torch.cuda.synchronize()
    ref, ref_o = _snap(d), _snap(o)
    g = csa2.capture_graph([d])
    for it in range(4):
        for t in (d.out, d.lse, d.sel_idx, d.kept):
            t.fill_(-7)          # poison: every replay must rewrite its outputs
        torch.cuda.synchronize()
        g.replay()
        if it % 2:
            o.run()              # eager work between replays
        torch.cuda.synchronize()
        for a, b in zip(_snap(d), ref):
            assert torch.equal(a, b), f"replay {it} differs from eager"
    for a, b in zip(_snap(o), ref_o):
        assert torch.equal(a, b)


def test_concurrent_streams_with_own_workspaces(csa2):
    # The entry points keep no state and allocate nothing, so two decoders (each with its
    # own outputs and workspace) enqueued on two streams at once give the results each
    # gives alone.
    wa, wb = make_config(2), make_config(3)
    da, db = upload(wa), upload(wb)
    a = csa2.Decoder(*da.decode_inputs(), sm_scale=wa.sm_scale)
    b = csa2.Decoder(*db.decode_inputs(), sm_scale=wb.sm_scale)
    a.run()
    b.run()
    torch.cuda.synchronize()
    ref_a, ref_b = _snap(a), _snap(b)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        for d in (a, b):
            for t in (d.out, d.lse, d.sel_idx, d.kept):
                t.fill_(-7)
        torch.cuda.synchronize()
        for _ in range(4):
            a.run(stream=sa.cuda_stream)
            b.run(stream=sb.cuda_stream)
        torch.cuda.synchronize()
        for x, y in zip(_snap(a), ref_a):
            assert torch.equal(x, y)
        for x, y in zip(_snap(b), ref_b):
            assert torch.equal(x, y)
