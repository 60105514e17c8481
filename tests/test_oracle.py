"""Pins for the oracle's scoring, selection and attention against brute force, library
routines, closed forms and invariants (no GPU)."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from synth import make_workload

E2M1_FRAC = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
             Fraction(6)]


def _fp4_record_fractions(rec, dim, block):
    """Independent exact decode: nibble values from the OCP table, scales via torch's E8M0."""
    scales = torch.from_numpy(rec[dim // 2:].copy()).view(torch.float8_e8m0fnu).double().tolist()
    out = []
    for j in range(dim):
        byte = int(rec[j // 2])
        c = (byte >> 4) if j % 2 else (byte & 15)
        v = E2M1_FRAC[c & 7] * Fraction(scales[j // block])
        out.append(-v if c & 8 else v)
    return out


def _bf16_fractions(bits):
    t = torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16).copy()).view(torch.bfloat16).double()
    return [Fraction(v) for v in t.flatten().tolist()]


@pytest.fixture(scope="module")
def tiny():
    # 3 requests: 130 entries (3 blocks, last partial), 64, 1 entry; 2 rows on the first.
    return make_workload("t", 123, [130, 64, 1], rows_per_req=[2, 1, 1], n_needles=4)


def test_index_score_bruteforce_exact(tiny):
    wl = tiny
    for r in range(wl.num_rows):
        b = int(wl.row_req[r])
        e0, e1 = int(wl.entry_off[b]), int(wl.entry_off[b + 1])
        q = _bf16_fractions(wl.q_idx[r])
        w = [Fraction(float(x)) for x in wl.w[r]]
        got = oracle.request_scores(wl, b)[r - int(wl.row_off[b])]
        for t in range(0, e1 - e0, 7):
            k = _fp4_record_fractions(wl.idx_k[e0 + t], 128, 32)
            s = Fraction(0)
            for h in range(8):
                dot = sum(q[h * 128 + d] * k[d] for d in range(128))
                s += w[h] * max(Fraction(0), dot)
            assert abs(got[t] - float(s)) <= 1e-12 * max(1.0, abs(float(s))), (r, t)


def test_block_score_bruteforce_exact(tiny):
    wl = tiny
    for r in range(wl.num_rows):
        b = int(wl.row_req[r])
        q = _bf16_fractions(wl.q_idx[r])
        w = [Fraction(float(x)) for x in wl.w[r]]
        got = oracle.block_scores_row(wl, r)
        for j in range(int(wl.block_off[b]), int(wl.block_off[b + 1])):
            k = _bf16_fractions(wl.blk_sum[j])
            s = sum(w[h] * max(Fraction(0), sum(q[h * 128 + d] * k[d] for d in range(128))) for h in range(8))
            assert abs(got[j - int(wl.block_off[b])] - float(s)) <= 1e-12 * max(1.0, abs(float(s)))


def test_index_score_single_head_is_relu_dot():
    rng = np.random.default_rng(3)
    q = np.zeros((8, 128))
    q[2] = rng.standard_normal(128)
    w = np.zeros(8)
    w[2] = 1.0
    keys = rng.standard_normal((50, 128))
    got = oracle.indexer_score(q, w, keys)
    ref = np.array([max(0.0, float(np.dot(q[2], k))) for k in keys])
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-14)


def _brute_topk(pos, sc, k):
    # Repeated selection of the best remaining (score desc, position asc).
    left = list(zip(pos.tolist(), sc.tolist()))
    out = []
    for _ in range(min(k, len(left))):
        best = None
        for i, (p, s) in enumerate(left):
            if best is None or s > left[best][1] or (s == left[best][1] and p < left[best][0]):
                best = i
        out.append(left.pop(best)[0])
    return sorted(out)


def test_topk_bruteforce_with_ties():
    rng = np.random.default_rng(5)
    for trial in range(40):
        n = int(rng.integers(1, 90))
        pos = np.sort(rng.choice(1000, size=n, replace=False))
        sc = rng.integers(0, 6, size=n).astype(np.float64)        # many exact ties
        k = int(rng.integers(1, 100))
        assert oracle.top_k(pos, sc, k).tolist() == _brute_topk(pos, sc, k)


def test_topk_k_at_least_candidates_returns_all():
    pos = np.array([5, 1, 9, 3])
    assert oracle.top_k(pos, np.array([0.1, 0.2, 0.3, 0.4]), 512).tolist() == [1, 3, 5, 9]


def test_keep_blocks_rules():
    # nb <= n_keep: identity.
    assert oracle.keep_blocks(np.arange(64.0), 64).tolist() == list(range(64))
    # The newest block is kept even with the lowest score.
    s = np.arange(100.0, 0.0, -1.0)                 # block 99 has the lowest score
    kept = oracle.keep_blocks(s, 64)
    assert kept.tolist() == list(range(64)) + [99]
    # Newest already in the top 64: exactly 64 kept.
    s2 = s.copy()
    s2[99] = 1000.0
    assert oracle.keep_blocks(s2, 64).tolist() == list(range(63)) + [99]
    # Ties go to the lower block.
    s3 = np.zeros(100)
    assert oracle.keep_blocks(s3, 64).tolist() == list(range(64)) + [99]
    assert oracle.keep_blocks(s3, 64, keep_newest=False).tolist() == list(range(64))


def test_keep_blocks_bruteforce():
    rng = np.random.default_rng(9)
    for _ in range(30):
        nb = int(rng.integers(1, 200))
        s = rng.integers(0, 10, size=nb).astype(float)
        ref = sorted(range(nb), key=lambda j: (-s[j], j))
        ref = set(ref[:64]) if nb > 64 else set(range(nb))
        ref.add(nb - 1)
        assert oracle.keep_blocks(s, 64).tolist() == sorted(ref)


def test_blocks_to_entries_partial_newest():
    assert oracle.blocks_to_entries(np.array([0, 2]), 130).tolist() == list(range(64)) + [128, 129]


def _sdpa(q, x, scale):
    # torch's reference attention in float64 on the CPU (K = V = x, one query per head).
    qt = torch.from_numpy(q)[None, :, None, :]              # [1, H, 1, D]
    kt = torch.from_numpy(x)[None, None].expand(1, q.shape[0], x.shape[0], x.shape[1])
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=scale)
    return o[0, :, 0].numpy()


def test_attention_matches_library_routines():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((64, 512))
    x = rng.standard_normal((300, 512))
    out, lse = oracle.joint_attention(q, x, 1 / math.sqrt(512))
    assert np.allclose(out, _sdpa(q, x, 1 / math.sqrt(512)), rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, scipy.special.logsumexp((q @ x.T) / math.sqrt(512), axis=1), rtol=1e-13)


def test_attention_closed_forms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((10, 512))
    # Single key: output is the key, lse is its logit.
    q = rng.standard_normal((64, 512))
    out, lse = oracle.joint_attention(q, x[:1], 0.1)
    assert np.allclose(out, np.broadcast_to(x[0], out.shape), rtol=0, atol=1e-15)
    assert np.allclose(lse, 0.1 * q @ x[0])
    # All-equal logits (q = 0): output is the mean of the keys, lse = log n.
    out, lse = oracle.joint_attention(np.zeros((64, 512)), x, 0.1)
    assert np.allclose(out, x.mean(axis=0)[None], atol=1e-14)
    assert np.allclose(lse, math.log(10))
    # No keys: zeros and -inf.
    out, lse = oracle.joint_attention(q, x[:0], 0.1)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_attention_lse_merge_and_permutation():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((64, 512))
    a = rng.standard_normal((40, 512))
    b = rng.standard_normal((25, 512)) * 2
    s = 1 / math.sqrt(512)
    oa, la = oracle.joint_attention(q, a, s)
    ob, lb = oracle.joint_attention(q, b, s)
    oj, lj = oracle.joint_attention(q, np.concatenate([a, b]), s)
    m = np.maximum(la, lb)
    wa, wb = np.exp(la - m), np.exp(lb - m)
    assert np.allclose(oj, (wa[:, None] * oa + wb[:, None] * ob) / (wa + wb)[:, None], rtol=1e-12, atol=1e-13)
    assert np.allclose(lj, m + np.log(wa + wb), rtol=1e-13)
    perm = rng.permutation(65)
    op, lp = oracle.joint_attention(q, np.concatenate([a, b])[perm], s)
    assert np.allclose(op, oj, rtol=1e-12, atol=1e-13) and np.allclose(lp, lj)


def test_decode_keep_all_equals_dense_attention():
    # With k >= N and the coarse stage keeping every block, the path is dense attention
    # over all of the request's entries plus the row's window.
    wl = make_workload("dense", 31, [300, 97], rows_per_req=[2, 1], n_needles=3, swa_len=[128, 40])
    res = oracle.decode(wl, k=4096, n_keep=1000)
    for r, rr in enumerate(res):
        b = int(wl.row_req[r])
        n = wl.n_entries(b)
        assert rr["sel"].tolist() == list(range(n))
        e0 = int(wl.entry_off[b])
        main = torch.from_numpy(wl.main_kv[e0:e0 + n].copy())
        # Independent decode of the main records via the OCP table and torch's E8M0/E4M3 decoders.
        x = np.array([[float(v) for v in _fp4_record_fractions(main[i].numpy(), 512, 16)] for i in range(n)])
        s0, sl = int(wl.row_swa_start[r]), int(wl.row_swa_len[r])
        win = torch.from_numpy(wl.swa[s0:s0 + sl].copy()).view(torch.float8_e4m3fn).double().numpy()
        win = win * wl.swa_scale[s0:s0 + sl].astype(np.float64)[:, None]
        keys = np.concatenate([x, win])
        q = torch.from_numpy(wl.q[r].view(np.int16).copy()).view(torch.bfloat16).double().numpy()
        assert np.allclose(rr["out"], _sdpa(q, keys, wl.sm_scale), rtol=1e-11, atol=1e-12)
        lse = scipy.special.logsumexp((q @ keys.T) * wl.sm_scale, axis=1)
        assert np.allclose(rr["lse"], lse, rtol=1e-12)


def test_decode_selection_composes_steps():
    # One row over 40 blocks with a small k: the oracle's selection equals brute force on
    # the candidates of its own coarse stage, and the coarse stage equals brute force on
    # block scores computed independently.
    wl = make_workload("sel", 77, [2560 + 17], rows_per_req=1, n_needles=8)
    rr = oracle.decode(wl, k=100, n_keep=10)[0]
    bs = oracle.block_scores_row(wl, 0)
    order = sorted(range(len(bs)), key=lambda j: (-bs[j], j))[:10]
    assert rr["kept"].tolist() == sorted(set(order) | {len(bs) - 1})
    cand = [t for t in range(wl.n_entries(0)) if t // 64 in set(rr["kept"].tolist())]
    assert rr["cand"].tolist() == cand
    assert rr["sel"].tolist() == _brute_topk(np.array(cand), rr["scores"][cand], 100)


def test_needles_rank_high_when_kept():
    # Needle keys are 3x the mean indexer query, so their scores exceed typical entries.
    wl = make_workload("needle", 5, [2048], rows_per_req=1, n_needles=16)
    rr = oracle.decode(wl)[0]
    assert set(wl.needles[0].tolist()) <= set(rr["sel"].tolist())


def test_empty_and_degenerate_requests():
    wl = make_workload("edge", 8, [0, 1, 63, 64, 65], rows_per_req=1, n_needles=1, swa_len=[0, 1, 128, 5, 0])
    res = oracle.decode(wl)
    assert res[0]["sel"].size == 0 and np.all(np.isneginf(res[0]["lse"]))
    assert res[1]["sel"].tolist() == [0]
    assert res[2]["sel"].tolist() == list(range(63))
    assert res[4]["kept"].tolist() == [0, 1] and res[4]["sel"].tolist() == list(range(65))
    for rr in res[1:]:
        assert np.all(np.isfinite(rr["out"])) and np.all(np.isfinite(rr["lse"]))


def test_generator_is_deterministic():
    a = make_workload("d", 3, [1000, 70], rows_per_req=[1, 2])
    b = make_workload("d", 3, [1000, 70], rows_per_req=[1, 2], workers=1)
    for f in ("idx_k", "main_kv", "blk_sum", "swa", "swa_scale", "q", "q_idx", "w"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


@pytest.mark.parametrize("i", [0])
def test_config0_oracle_runs(i):
    from synth import make_config
    wl = make_config(i)
    rr = oracle.decode(wl)[0]
    assert rr["sel"].size == 512 and rr["kept"].size == 32
    assert np.all(np.isfinite(rr["out"]))


# ---------------------------------------------------------------------------------
# Row visibility, score check and paged pools.
# ---------------------------------------------------------------------------------

def _truncated(wl, r, v):
    """Row r alone, over its request cut to its first v entries (arrays sliced here,
    independently of the oracle's row-visibility code)."""
    from synth import Workload
    b = int(wl.row_req[r])
    e0, b0 = int(wl.entry_off[b]), int(wl.block_off[b])
    nb = -(-v // 64)
    s0, sl = int(wl.row_swa_start[r]), int(wl.row_swa_len[r])
    return Workload(name="cut", seed=0, n_tokens=[v], entry_off=np.array([0, v], dtype=np.int64),
                    block_off=np.array([0, nb], dtype=np.int64), row_off=np.array([0, 1], dtype=np.int32),
                    swa_off=np.array([0, sl], dtype=np.int64), row_req=np.zeros(1, dtype=np.int32),
                    row_swa_start=np.zeros(1, dtype=np.int64), row_swa_len=np.array([sl], dtype=np.int32),
                    idx_k=wl.idx_k[e0:e0 + v], main_kv=wl.main_kv[e0:e0 + v], blk_sum=wl.blk_sum[b0:b0 + nb],
                    swa=wl.swa[s0:s0 + sl], swa_scale=wl.swa_scale[s0:s0 + sl], q=wl.q[r:r + 1],
                    q_idx=wl.q_idx[r:r + 1], w=wl.w[r:r + 1])


def test_row_len_equals_truncated_request():
    # A row that sees V entries decodes exactly like a request holding only those V.
    wl = make_workload("rl", 31, [64 * 90 + 17, 700], rows_per_req=[4, 2], n_needles=8)
    wl.row_len = np.array([64 * 90 + 17, 64 * 90, 64 * 70 + 1, 5000, 700, 1], dtype=np.int64)
    got = oracle.decode(wl, k=300, n_keep=40)
    for r in range(wl.num_rows):
        v = int(wl.row_len[r])
        ref = oracle.decode(_truncated(wl, r, v), k=300, n_keep=40)[0]
        assert got[r]["block_scores"].shape[0] == -(-v // 64)
        for key in ("kept", "sel", "out", "lse", "block_scores"):
            assert np.array_equal(got[r][key], ref[key]), (r, key)
        assert got[r]["sel"].size == 0 or got[r]["sel"].max() < v


def test_row_len_zero_and_beyond():
    wl = make_workload("rl0", 32, [300], rows_per_req=[3], n_needles=2)
    wl.row_len = np.array([0, 10 ** 9, -4], dtype=np.int64)   # clamps to 0 .. N
    got = oracle.decode(wl)
    assert got[0]["sel"].size == 0 and got[0]["kept"].size == 0 and got[2]["sel"].size == 0
    full = oracle.decode(make_workload("rl0", 32, [300], rows_per_req=[3], n_needles=2))
    assert np.array_equal(got[1]["sel"], full[1]["sel"]) and np.array_equal(got[1]["out"], full[1]["out"])
    # No main entries: attention over the window alone.
    ro, rl = oracle.joint_attention(oracle.bf16_value(wl.q[0]), oracle.row_keys(wl, 0, np.zeros(0)), wl.sm_scale)
    assert np.array_equal(got[0]["out"], ro) and np.array_equal(got[0]["lse"], rl)


def _is_topk(positions, scores, k, sel):
    """True iff ``sel`` is the unique set of min(k, #non-NaN) non-NaN candidates such that
    every pick beats every non-pick by (score desc, position asc)."""
    valid = {int(t): float(s) for t, s in zip(positions, scores) if not math.isnan(s)}
    sel = [int(t) for t in sel]
    if len(set(sel)) != len(sel) or any(t not in valid for t in sel) or len(sel) != min(k, len(valid)):
        return False
    rest = set(valid) - set(sel)
    return all(valid[s] > valid[u] or (valid[s] == valid[u] and s < u) for s in sel for u in rest)


def test_topk_skips_nan_scores():
    rng = np.random.default_rng(5)
    for trial in range(40):
        n = int(rng.integers(1, 60))
        pos = np.sort(rng.choice(1000, size=n, replace=False))
        sc = rng.integers(-3, 4, size=n).astype(np.float64)
        sc[rng.random(n) < 0.3] = np.nan
        for k in (1, 3, n // 2 + 1, n, n + 5):
            sel = oracle.top_k(pos, sc, k)
            assert np.all(np.diff(sel) > 0)
            assert _is_topk(pos, sc, k, sel), (trial, k)
    assert oracle.top_k(np.arange(4), np.full(4, np.nan), 2).size == 0


def test_keep_blocks_skips_nan_scores():
    rng = np.random.default_rng(6)
    for trial in range(40):
        nb = int(rng.integers(1, 40))
        bs = rng.integers(0, 5, size=nb).astype(np.float64)
        bs[rng.random(nb) < 0.3] = np.nan
        for n_keep in (1, 4, nb):
            for newest in (True, False):
                kept = oracle.keep_blocks(bs, n_keep, newest).tolist()
                # Either the kept set is the ranked top set itself, or (newest rule) the
                # top set plus the newest block that the ranking left out.
                ok = _is_topk(np.arange(nb), bs, n_keep, kept)
                if not ok and newest and kept and kept[-1] == nb - 1:
                    ok = _is_topk(np.arange(nb), bs, n_keep, kept[:-1])
                assert ok, (trial, n_keep, newest)
                assert (nb - 1 in kept) or not newest
                assert np.all(np.diff(kept) > 0)


def test_decode_never_selects_nan_scored_entries():
    # Entries with an E8M0 NaN scale byte score NaN; the needles (which would rank first)
    # are given one, so the selection must fall back to the other entries.
    wl = make_workload("nan", 33, [64 * 80 + 9], rows_per_req=[2], n_needles=16)
    bad = wl.needles[0]
    wl.idx_k[bad, 64] = 255
    got = oracle.decode(wl, k=200, n_keep=20)
    for r in range(2):
        s = got[r]["scores"]
        assert np.all(np.isnan(s[bad]))
        assert not set(bad.tolist()) & set(got[r]["sel"].tolist())
        assert _is_topk(got[r]["cand"], got[r]["cand_scores"], 200, got[r]["sel"])
    # A block summary scoring NaN is never ranked, but the newest-block rule still keeps
    # the newest block.
    wl.blk_sum[[3, 80]] = 0x7FC0
    got = oracle.decode(wl, k=200, n_keep=20)
    for r in range(2):
        assert 3 not in got[r]["kept"] and 80 in got[r]["kept"]


def test_paged_pools_match_contiguous():
    # Pages scattered over a pool with spare pages of random bytes: reading any row the
    # page table does not name changes the result.
    from synth import to_paged
    wl = make_workload("pg", 34, [64 * 40 + 5, 1000, 64, 1, 0], rows_per_req=[1, 3, 2, 1, 1], n_needles=6)
    pw = to_paged(wl)
    assert pw.page_table.shape == (5, 41) and pw.total_pages > 41 + 16 + 1 + 1
    assert len(set(pw.page_table[pw.page_table >= 0].tolist())) == int((pw.page_table >= 0).sum())
    a, b = oracle.decode(wl, k=300, n_keep=16), oracle.decode(pw, k=300, n_keep=16)
    for r, (x, y) in enumerate(zip(a, b)):
        for key in ("kept", "sel", "out", "lse", "block_scores", "scores"):
            assert np.array_equal(x[key], y[key]), (r, key)
    # The page table is what locates the data: a swapped pair of pages changes the keys.
    pw.page_table[1, [0, 1]] = pw.page_table[1, [1, 0]]
    c = oracle.decode(pw, rows=[1], k=300, n_keep=16)[0]
    assert not np.array_equal(c["scores"], a[1]["scores"])


# ---------------------------------------------------------------------------------
# MXFP8 route.
# ---------------------------------------------------------------------------------

def _mx_reference(x):
    """Independent MXFP8 rounding of one 32-value block: shared exponent from frexp,
    elements through torch's float8_e4m3fn conversion (round to nearest even), values
    above 448 clamped first (saturation)."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max()
    if amax == 0:
        return np.zeros_like(x)
    s = max(-127, min(127, int(np.floor(np.log2(amax))) - 8))
    y = np.clip(x / 2.0 ** s, -448.0, 448.0)
    e = torch.from_numpy(y).to(torch.float8_e4m3fn).double().numpy()
    return e * 2.0 ** s


def test_mxfp8_round_matches_torch_e4m3():
    rng = np.random.default_rng(11)
    blocks = []
    for mag in (1e-30, 1e-6, 2.0 ** -20, 0.1, 1.0, 3.7, 448.0, 1e5, 2.0 ** 100):
        for _ in range(20):
            blocks.append(rng.standard_normal(32) * mag)
    b = rng.standard_normal(32)
    b[3] = 0.0
    b[5] = b.max() * 1e-6                      # deep in E4M3's subnormal range
    blocks.append(b)
    blocks.append(np.zeros(32))
    x = np.stack(blocks)
    got = oracle.mxfp8_round(x)
    ref = np.stack([_mx_reference(v) for v in x])
    assert np.array_equal(got, ref)


def test_mxfp8_round_closed_forms():
    # Block max 500: scale 2^0.  Ties go to the even code; above 448 saturates.
    x = np.zeros(32)
    x[:9] = [17.0, 19.0, 300.0, 500.0, 460.0, -17.0, 0.0009765625, 0.00146484375, 0.5]
    got = oracle.mxfp8_round(x)[:9]
    assert got.tolist() == [16.0, 20.0, 288.0, 448.0, 448.0, -16.0, 0.0, 0.001953125, 0.5]
    # Values already on an MX grid are unchanged; a scale of 2^k leaves the codes alone.
    y = oracle.mxfp8_round(np.linspace(-3, 3, 64))
    assert np.array_equal(oracle.mxfp8_round(y), y)
    assert np.array_equal(oracle.mxfp8_round(y * 2.0 ** 40), y * 2.0 ** 40)
    # Partial last block is padded for the scale only.
    assert oracle.mxfp8_round(np.array([1.0, 17.0])).tolist() == [1.0, 16.0]


def test_mx_attention_closed_forms_and_bound():
    rng = np.random.default_rng(12)
    codes = oracle.E2M1[rng.integers(0, 16, size=(70, 512))]
    # Equal logits (q = 0): p = 1 everywhere, MXFP8(1) = 1, so out is the plain mean.
    q = np.zeros((64, 512))
    out, lse = oracle.joint_attention_mx(q, codes, np.ones(70), 0.05)
    assert np.allclose(out, codes.mean(axis=0)[None, :], rtol=0, atol=1e-12)
    assert np.allclose(lse, np.log(70.0))
    # With unrounded Q and P the route is the plain attention; rounding moves the output
    # by no more than the bound it reports.
    q = oracle.mxfp8_round(rng.standard_normal((64, 512)))   # already on the MX grid
    sc = np.ones(70)
    o1, l1, bound = oracle.joint_attention_mx(q, codes, sc, 0.04, with_bound=True)
    o0, l0 = oracle.joint_attention(q, codes, 0.04)
    assert np.allclose(l1, l0, rtol=0, atol=1e-12)
    assert np.all(np.abs(o1 - o0) <= bound / 2 + 1e-12)
    assert np.abs(o1 - o0).max() > 0        # P really is rounded


def test_mx_attention_rounds_p_in_blocks_of_keys():
    # The expected output is built head by head and key block by key block (32
    # consecutive keys, a partial last block of 8) with the independent rounding above:
    # q rounded per head in blocks of 32 dims, the weight on each key's codes
    # w_i = p_i * scale_i rounded per head in blocks of keys, normaliser and lse from the
    # unrounded p.  Rounding the weights along heads instead (blocks of 32 heads per key)
    # gives a clearly different output on the same data.
    rng = np.random.default_rng(13)
    n, H, sm = 40, 64, 0.07
    codes = oracle.E2M1[rng.integers(0, 16, size=(n, 512))]
    scales = np.ones(n)
    scales[-8:] = rng.uniform(0.01, 0.1, 8)          # the last keys act as scaled window tokens
    q = rng.standard_normal((H, 512)) * 0.5
    blocks = [(0, 32), (32, 40)]
    qm = np.stack([np.concatenate([_mx_reference(q[h, 32 * j:32 * j + 32]) for j in range(16)]) for h in range(H)])
    want = np.zeros((H, 512))
    want_lse = np.zeros(H)
    w_all = np.zeros((H, n))
    l_all = np.zeros(H)
    for h in range(H):
        z = np.array([sm * scales[i] * float(qm[h] @ codes[i]) for i in range(n)])
        mz = z.max()
        p = np.exp(z - mz)
        w = p * scales
        w_all[h], l_all[h] = w, p.sum()
        wr = np.concatenate([_mx_reference(w[a:b]) for a, b in blocks])
        want[h] = (wr[:, None] * codes).sum(axis=0) / p.sum()
        want_lse[h] = mz + np.log(p.sum())
    out, lse = oracle.joint_attention_mx(q, codes, scales, sm)
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, want_lse, rtol=0, atol=1e-12)
    by_heads = np.stack([np.concatenate([_mx_reference(w_all[a:b, i]) for a, b in ((0, 32), (32, 64))])
                         for i in range(n)], axis=1)
    other = (by_heads @ codes) / l_all[:, None]
    assert np.abs(other - want).max() > 1e-3 * np.abs(want).max()


# ---------------------------------------------------------------------------------
# Cache write.
# ---------------------------------------------------------------------------------

def test_fp4_encode_matches_the_input_generators_encoder():
    # Two independent encoders of the same OCP MX rule (the generator's uses threshold
    # counts, the oracle's nearest-value search).
    from synth.generator import encode_fp4_blocks
    rng = np.random.default_rng(40)
    x = (rng.standard_normal((200, 512)) * np.exp(rng.uniform(-20, 20, size=(200, 1)))).astype(np.float32)
    x[0] = 0.0
    x[1, :16] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75, 0.0, 4.5, 5.5, 1e-30, -1.0, 0.1]
    x[2, :32] = np.ldexp(np.arange(32) / 4.0, -3)          # every E2M1 midpoint at scale 2^-3
    for block in (16, 32):
        got = oracle.pack_fp4_record(*oracle.fp4_encode(x, block))
        assert np.array_equal(got, encode_fp4_blocks(x, block)), block
    # Round trip: values on the grid come back unchanged.
    codes, exps = oracle.fp4_encode(x, 16)
    rec = oracle.pack_fp4_record(codes, exps)
    back = oracle.dequant_fp4_records(rec, 512, 16)
    again = oracle.pack_fp4_record(*oracle.fp4_encode(back, 16))
    assert np.array_equal(again, rec)


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(41)
    x = rng.standard_normal(5000).astype(np.float32).astype(np.float64)   # fp32-exact inputs
    x[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 3.0]
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_rne(x), ref)


def _write_case(seed, lens, rows, last_even=True):
    from synth import make_workload, make_write_inputs
    wl = make_workload("w", seed, lens, rows_per_req=rows, n_needles=2)
    w = make_write_inputs(wl, seed + 1, last_even)
    return (wl, w["row_pos"], w["kv_tok"], w["idx_tok"], w["ring_kv"], w["ring_idx"], w["gamma_kv"],
            w["gamma_idx"])


def test_cache_write_rules():
    wl, pos, kv, ik, rkv, ridx, gk, gi = _write_case(42, [300, 64 * 5], [5, 6])
    res = oracle.cache_write(wl, pos, kv, ik, rkv, ridx, gk, gi)
    # Entries written: odd positions only, below N_b.
    assert sorted(res["written"]) == sorted((b, (int(p) - 1) // 2) for r, p in enumerate(pos) if p % 2 == 1
                                            for b in [int(wl.row_req[r])] if (int(p) - 1) // 2 < wl.n_entries(b))
    # Rows not written are untouched.
    changed = np.flatnonzero((res["idx_k"] != wl.idx_k).any(axis=1) | (res["main_kv"] != wl.main_kv).any(axis=1))
    rows = {int(oracle.entry_rows(wl, b, np.array([t]))[0]) for (b, t) in res["written"]}
    assert set(changed.tolist()) <= rows
    # The pooling partner of a request's first row (here request 1: 6 rows ending at
    # 2 N_b start at an odd position) is its ring slot; the same token as an extra row
    # just before it gives the same records.
    b = 1
    r0 = int(wl.row_off[b])
    assert pos[r0] % 2 == 1
    kv2 = np.concatenate([kv[:r0], rkv[b:b + 1], kv[r0:]])
    ik2 = np.concatenate([ik[:r0], ridx[b:b + 1], ik[r0:]])
    wl2 = type(wl)(**{f: getattr(wl, f) for f in wl.__dataclass_fields__})
    wl2.row_off = wl.row_off + np.array([0, 0, 1], dtype=np.int32)
    wl2.row_req = np.concatenate([wl.row_req[:r0], [b], wl.row_req[r0:]]).astype(np.int32)
    pos2 = np.concatenate([pos[:r0], [pos[r0] - 1], pos[r0:]])
    kv2_ring, ik2_ring = rkv.copy(), ridx.copy()
    kv2_ring[b] = 0
    ik2_ring[b] = 0
    res2 = oracle.cache_write(wl2, pos2, kv2, ik2, kv2_ring, ik2_ring, gk, gi)
    assert np.array_equal(res2["main_kv"], res["main_kv"]) and np.array_equal(res2["idx_k"], res["idx_k"])
    # Summaries: bf16 of the mean of the block's dequantised keys.
    t = max(t for (bb, t) in res["written"] if bb == 1)
    j = t // 64
    keys = oracle.dequant_idx(res["idx_k"][oracle.entry_rows(wl, 1, np.arange(64 * j, min(64 * j + 64, 320)))])
    assert np.array_equal(res["blk_sum"][int(wl.block_off[1]) + j], oracle.bf16_rne(keys.mean(axis=0)))
    # The last row of request 1 (position 2 N_b, even) went to its ring slot.
    assert np.array_equal(res["ring_kv"][1], kv[int(wl.row_off[2]) - 1])


def test_cache_write_is_scale_invariant():
    # RMSNorm: scaling both pooled tokens by a power of two leaves every record alone.
    wl, pos, kv, ik, rkv, ridx, gk, gi = _write_case(43, [200], [4])
    a = oracle.cache_write(wl, pos, kv, ik, rkv, ridx, gk, gi, eps=1e-30)
    up = lambda bits: (bits.astype(np.uint32) + (3 << 7)).astype(np.uint16)   # x 8 in bf16 (exponent + 3)
    b = oracle.cache_write(wl, pos, up(kv), up(ik), up(rkv), up(ridx), gk, gi, eps=1e-30)
    assert np.array_equal(a["main_kv"], b["main_kv"]) and np.array_equal(a["idx_k"], b["idx_k"])
    # Doubling gamma doubles every value: same codes, every scale byte one higher.
    c = oracle.cache_write(wl, pos, kv, ik, rkv, ridx, gk * 2, gi * 2, eps=1e-30)
    for (bb, t) in a["written"]:
        row = int(oracle.entry_rows(wl, bb, np.array([t]))[0])
        assert np.array_equal(c["main_kv"][row, :256], a["main_kv"][row, :256])
        assert np.array_equal(c["main_kv"][row, 256:].astype(int), a["main_kv"][row, 256:].astype(int) + 1)


def test_rms_norm_closed_forms():
    # y = x * gamma / sqrt(mean(x^2) + eps), per row.  A sum in place of the mean, eps
    # outside the square root, or gamma applied as a scalar each fail one of these.
    assert np.allclose(oracle.rms_norm(np.array([[3.0, 4.0]]), np.ones(2), 0.0),
                       [[3 * math.sqrt(2) / 5, 4 * math.sqrt(2) / 5]], rtol=0, atol=1e-15)
    assert np.allclose(oracle.rms_norm(np.ones((1, 4)), np.ones(4), 3.0), 0.5, rtol=0, atol=1e-15)
    assert np.allclose(oracle.rms_norm(np.array([[2.0, 2.0]]), np.array([1.0, 3.0]), 0.0), [[1.0, 3.0]],
                       rtol=0, atol=1e-15)
    assert np.allclose(oracle.rms_norm(np.array([[1.0, 1.0], [-2.0, 2.0]]), np.ones(2), 0.0),
                       [[1.0, 1.0], [-1.0, 1.0]], rtol=0, atol=1e-15)
    # eps dominates a tiny vector: y = x / sqrt(eps)
    assert np.allclose(oracle.rms_norm(np.full((1, 8), 1e-9), np.ones(8), 1e-2), 1e-8, rtol=1e-9, atol=0)


def test_cache_write_golden_record():
    # A token pair with distinct partner and own vectors, its main and index records and
    # block summary derived by hand (tests/golden/cache_write_record.json).  Pooling that
    # ignored the partner, RMSNorm over a sum, or a wrong code/scale rule all change them.
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cache_write_record.json")))

    def bf16_vec(nonzero, dim):
        v = np.zeros(dim, dtype=np.float32)
        for k, x in nonzero.items():
            v[int(k)] = x
        return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)[None]

    wl = make_workload("golden", 5, [1], rows_per_req=1, n_needles=0)
    res = oracle.cache_write(wl, np.array([1]), bf16_vec(g["kv_tok_nonzero"], 512),
                             bf16_vec(g["idx_tok_nonzero"], 128), bf16_vec(g["ring_kv_nonzero"], 512),
                             bf16_vec(g["ring_idx_nonzero"], 128), np.ones(512), np.ones(128), eps=g["eps"])
    for pool, key, width in (("main_kv", "main_expected", 288), ("idx_k", "index_expected", 68),
                             ("blk_sum", "summary_expected", 128)):
        want = np.zeros(width, dtype=np.int64)
        for k, v in g[key].items():
            want[int(k)] = v
        assert np.array_equal(res[pool][0].astype(np.int64), want), pool
    assert sorted(res["written"]) == [(0, 0)]
