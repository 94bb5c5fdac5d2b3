"""Comparison rules between the GPU library and the CPU oracle.

Selection indices are integers decided by floating-point scores, and several answers are
correct when two candidates' scores are within rounding of each other.  The rule:
  * a row (b, t, g) is a NEAR-TIE row when any adjacent gap among the oracle's top
    min(K+1, n_avail) sorted scores is below 1e-4;
  * outside near-tie rows the GPU's idx must equal the oracle's bit for bit (order and -1s);
  * on near-tie rows whose idx differ, the GPU's choice must still be a valid top-K: the same
    number of valid slots, distinct causal chunks, and each slot's oracle score within 1e-4 of
    the oracle's score for that rank;
  * scores and weights are compared (1e-5) and outputs element by element on every row whose
    idx agree; rows whose idx differ are counted and reported.
"""
from __future__ import annotations

import numpy as np

NEAR_TIE = 1e-4
SCORE_TOL = 1e-5


def tol_for(dtype) -> float:
    import torch
    return 1e-4 if dtype == torch.float32 else 2e-2


def near_tie_rows(orc, Qs, Kslc_or, S, K, sel_scale=None, row_mask=None):
    _, sc, _ = orc.select(Qs, Kslc_or, S, K + 1, sel_scale=sel_scale, row_mask=row_mask)
    a, b = sc[..., :-1], sc[..., 1:]
    valid = np.isfinite(a) & np.isfinite(b)
    gap = np.where(valid, a - b, np.inf)
    return (gap < NEAR_TIE).any(-1)


def oracle_scores_of(Qs, Kslc_or, idx, sel_scale):
    """Oracle-precision scores (fp64 dot of stored values, rounded to fp32) of given chunks."""
    qs = Qs.double().cpu().numpy() if hasattr(Qs, "double") else np.asarray(Qs, np.float64)
    B, L, Hkv, D = qs.shape
    out = np.full(idx.shape, -np.inf)
    bb, tt, gg, kk = np.nonzero(idx >= 0)
    cc = idx[bb, tt, gg, kk]
    dots = np.einsum("nd,nd->n", qs[bb, tt, gg], Kslc_or[bb, cc, gg])
    out[bb, tt, gg, kk] = (sel_scale * dots).astype(np.float32).astype(np.float64)
    return out


def check_selection(gpu, orc_out, near, Qs, Kslc_or, S, sel_scale, row_mask=None):
    """gpu / orc_out: dicts with idx, score, w (numpy).  Returns (rows_differing mask, report)."""
    gi, oi = gpu["idx"], orc_out["idx"]
    rows = np.ones(gi.shape[:-1], bool) if row_mask is None else np.broadcast_to(
        np.asarray(row_mask, bool).reshape(gi.shape[0], gi.shape[1], 1), gi.shape[:-1])
    diff = (gi != oi).any(-1) & rows
    bad = diff & ~near
    assert not bad.any(), f"{int(bad.sum())} non-near-tie rows differ, first at {np.argwhere(bad)[:3]}"
    if diff.any():
        # the GPU's choice must be a valid top-K within the tie tolerance
        sg = oracle_scores_of(Qs, Kslc_or, np.where(diff[..., None], gi, -1), sel_scale)
        for (b, t, g) in np.argwhere(diff):
            nv_g = int((gi[b, t, g] >= 0).sum())
            nv_o = int((oi[b, t, g] >= 0).sum())
            assert nv_g == nv_o, (b, t, g, gi[b, t, g], oi[b, t, g])
            ch = gi[b, t, g, :nv_g]
            assert len(set(ch.tolist())) == nv_g, (b, t, g, ch)
            assert nv_g == 0 or ch.max() < t // S, (b, t, g, ch)
            assert np.all(np.abs(sg[b, t, g, :nv_g] - orc_out["score"][b, t, g, :nv_o]) < NEAR_TIE)
    same = rows & ~diff
    for key in ("score", "w"):
        g_, o_ = gpu[key][same], orc_out[key][same]
        fin = np.isfinite(o_)
        assert np.array_equal(np.isfinite(g_), fin), key
        if fin.any():
            err = np.abs(g_[fin] - o_[fin]).max()
            assert err <= SCORE_TOL, (key, err)
    report = dict(rows=int(rows.sum()), near_tie_rows=int((near & rows).sum()),
                  differing_rows=int(diff.sum()))
    return diff, report


def max_abs(a, b, mask=None):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    d = np.abs(a - b)
    if mask is not None:
        d = d[mask]
    return float(d.max()) if d.size else 0.0
