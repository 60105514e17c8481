"""Comparison of an implementation's decode results with the oracle (test infrastructure).

Rules (restated; the tolerances are those fixed for this path):
  * kept blocks: equal to the oracle's, except blocks whose oracle block score lies
    within ``rel`` of the oracle's n_keep-th best block score (the coarse boundary);
    the fine stage is then judged against the oracle re-run on the implementation's
    kept blocks;
  * selected set: equal to the oracle's, except positions whose oracle score lies within
    ``rel`` (1e-5) relative of the k-th best candidate score;
  * attention: max over (head, dim) of |O - O_ref| / max_dim |O_ref[head]| <= 2e-3 and
    |lse - lse_ref| <= 2e-3, against the oracle re-run on the implementation's own
    selected set (always) and against the oracle's own set when the sets are equal.
"""
from __future__ import annotations

import numpy as np

from . import csa2_oracle as O

SET_REL = 1e-5
ATTN_REL = 2e-3
LSE_ABS = 2e-3


def kth_best(scores: np.ndarray, k: int) -> float:
    """k-th best of the scores that are not NaN (NaN scores are never ranked)."""
    s = np.asarray(scores, dtype=np.float64)
    s = s[~np.isnan(s)]
    if s.size == 0:
        return 0.0
    k = min(k, s.size)
    return float(np.sort(s)[::-1][k - 1])


def band_ok(diff_positions, score_of, boundary: float, rel: float) -> tuple[bool, str]:
    for t in diff_positions:
        s = float(score_of(t))
        if np.isnan(s) or abs(s - boundary) > rel * abs(boundary):
            return False, f"position {t} (score {s!r}) differs but is outside the band around {boundary!r}"
    return True, ""


def attn_error(out, lse, out_ref, lse_ref) -> tuple[float, float]:
    """(max relative error normalised per head, max |lse error|); both 0 for matching empties."""
    out = np.asarray(out, dtype=np.float64)
    out_ref = np.asarray(out_ref, dtype=np.float64)
    den = np.abs(out_ref).max(axis=-1, keepdims=True)
    den = np.where(den > 0, den, 1.0)
    rel = float((np.abs(out - out_ref) / den).max()) if out.size else 0.0
    lse = np.asarray(lse, dtype=np.float64)
    lse_ref = np.asarray(lse_ref, dtype=np.float64)
    both_inf = np.isneginf(lse) & np.isneginf(lse_ref)
    d = np.where(both_inf, 0.0, np.abs(lse - lse_ref))
    return rel, float(np.nan_to_num(d, nan=np.inf).max()) if d.size else 0.0


def check_row(wl, r: int, ref: dict, kept_gpu: np.ndarray | None, sel_gpu: np.ndarray, out_gpu: np.ndarray,
              lse_gpu: np.ndarray, k: int | None = None, n_keep: int | None = None) -> dict:
    """Judge one row; returns a report dict with ``ok`` and the measured errors."""
    k = wl.k if k is None else k
    n_keep = wl.n_keep if n_keep is None else n_keep
    rep = {"row": r, "ok": True, "msgs": []}
    n = O.visible(wl, r)

    # Coarse stage.
    kept_ref = ref["kept"]
    kept = kept_ref
    if kept_gpu is not None:
        kept_gpu = np.asarray(kept_gpu, dtype=np.int64)
        rep["kept_equal"] = bool(np.array_equal(kept_gpu, kept_ref))
        if not rep["kept_equal"]:
            bs = ref["block_scores"]
            boundary = kth_best(bs, n_keep)
            diff = set(kept_gpu.tolist()) ^ set(kept_ref.tolist())
            ok, msg = band_ok(sorted(diff), lambda j: bs[j], boundary, SET_REL)
            if not ok:
                rep["ok"] = False
                rep["msgs"].append("kept blocks: " + msg)
            kept = kept_gpu
    # Fine stage against the oracle run on the kept blocks actually used.
    cand = O.blocks_to_entries(kept, n)
    cs = ref["scores"][cand]
    sel_ref = O.top_k(cand, cs, k) if kept is not kept_ref else ref["sel"]
    sel_gpu = np.asarray(sel_gpu, dtype=np.int64)
    rep["set_equal"] = bool(np.array_equal(np.sort(sel_gpu), sel_ref))
    rep["sel_sorted"] = bool(np.all(np.diff(sel_gpu) > 0)) if sel_gpu.size > 1 else True
    if not rep["sel_sorted"]:
        rep["ok"] = False
        rep["msgs"].append("selected positions are not strictly ascending")
    if not rep["set_equal"]:
        boundary = kth_best(cs, k)
        score_of = {t: v for t, v in zip(cand.tolist(), cs.tolist()) if not np.isnan(v)}
        diff = set(sel_gpu.tolist()) ^ set(sel_ref.tolist())
        outside = [t for t in diff if t not in score_of]
        if outside:
            rep["ok"] = False
            rep["msgs"].append(f"selected positions outside the candidates: {outside[:5]}")
        else:
            ok, msg = band_ok(sorted(diff), lambda t: score_of[t], boundary, SET_REL)
            if not ok:
                rep["ok"] = False
                rep["msgs"].append("selected set: " + msg)
        if sel_gpu.size != sel_ref.size:
            rep["ok"] = False
            rep["msgs"].append(f"selected {sel_gpu.size} positions, oracle {sel_ref.size}")
    # Attention on the implementation's own set (always).
    out_own, lse_own = O.joint_attention(O.bf16_value(wl.q[r]), O.row_keys(wl, r, sel_gpu), wl.sm_scale)
    rel, dl = attn_error(out_gpu, lse_gpu, out_own, lse_own)
    rep["attn_rel_own"], rep["lse_err_own"] = rel, dl
    if not (rel <= ATTN_REL and dl <= LSE_ABS):
        rep["ok"] = False
        rep["msgs"].append(f"attention vs oracle on own set: rel {rel:.3g}, lse {dl:.3g}")
    if rep["set_equal"] and kept is kept_ref:
        rel2, dl2 = attn_error(out_gpu, lse_gpu, ref["out"], ref["lse"])
        rep["attn_rel_ref"], rep["lse_err_ref"] = rel2, dl2
        if not (rel2 <= ATTN_REL and dl2 <= LSE_ABS):
            rep["ok"] = False
            rep["msgs"].append(f"attention vs oracle: rel {rel2:.3g}, lse {dl2:.3g}")
    return rep
