"""Comparison rules between the GPU library and the CPU oracle.

Selection indices are integers decided by floating-point scores, and several answers are
correct when two candidates' scores are within rounding of each other.  The rule:
  * a row (b, t, g) is a NEAR-TIE row when any adjacent gap among the oracle's top
    min(K+1, n_avail) sorted scores is below 1e-4;
  * outside near-tie rows the GPU's idx must equal the oracle's bit for bit (order and -1s);
  * on near-tie rows whose idx differ, the GPU's choice must still be a valid top-K: the same
    number of valid slots, distinct causal chunks, and each slot's oracle score within 1e-4 of
    the oracle's score for that rank;
  * scores and weights are compared (1e-5) on every row whose idx agree; rows whose idx
    differ are counted and reported;
  * outputs and gradients are compared element by element on every row and chunk, against
    the oracle evaluated on the GPU's own selection (idx, score, w), so a near-tie that was
    resolved the other way is checked like any other row.
"""
from __future__ import annotations

import numpy as np
import torch

NEAR_TIE = 1e-4
SCORE_TOL = 1e-5


def tol_for(dtype) -> float:
    import torch
    return 1e-4 if dtype == torch.float32 else 2e-2


def near_tie_rows(orc, Qs, Kslc_or, S, K, sel_scale=None, row_mask=None):
    _, sc, _ = orc.select(Qs, Kslc_or, S, K + 1, sel_scale=sel_scale, row_mask=row_mask)
    a, b = sc[..., :-1], sc[..., 1:]
    valid = np.isfinite(a) & np.isfinite(b)
    gap = np.full(a.shape, np.inf)
    np.subtract(a, b, out=gap, where=valid)  # masked slots (-inf) never enter the subtraction
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


def say(*a):
    print(*a, flush=True)


def npy(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def head_mask(row_mask_bLg, G):
    """[B, L, Hkv] -> [B, L, Hkv*G] (query head h belongs to group h // G)."""
    return np.repeat(row_mask_bLg, G, axis=2)


def compare_forward(orc, x, wl, g, row_mask=None, out_mask=None, weights="stick"):
    """Selection on the rows of row_mask (default: all), outputs on those of out_mask
    (default: row_mask).  The selection is compared with the oracle's own (bit-exact outside
    near-tie rows, a valid top-K on the near-tie rows that differ); O is compared on every
    asked row against the oracle's attention over the GPU's own selection (idx and w), so a
    row whose near-tie resolved differently is checked like any other."""
    Kslc = orc.pool(x["K"], wl.S)
    idx, score, w = orc.select(x["Qs"], Kslc, wl.S, wl.K, row_mask=row_mask, weights=weights)
    f = dict(Kslc=Kslc, idx=idx, score=score, w=w)
    near = near_tie_rows(orc, x["Qs"], Kslc, wl.S, wl.K, row_mask=row_mask)
    assert np.array_equal(npy(g["Kslc"]), Kslc), "pooled chunk keys differ"
    gpu = dict(idx=npy(g["idx"]), score=npy(g["score"]), w=npy(g["w"]))
    diff, rep = check_selection(gpu, f, near, x["Qs"], Kslc, wl.S, 1.0 / np.sqrt(wl.D),
                                row_mask)
    om = row_mask if out_mask is None else out_mask
    f["O"] = orc.attend(x["Q"], x["K"], x["V"], gpu["idx"], gpu["w"], wl.S, row_mask=om)
    keep = None
    if om is not None:
        keep = head_mask(np.broadcast_to(np.asarray(om, bool).reshape(wl.B, wl.L, 1),
                                         diff.shape), wl.G)
    err = max_abs(npy(g["O"]), f["O"], keep)
    rep["O_max_abs"] = err
    say("forward", wl.name, rep)
    assert err <= tol_for(wl.dtype), err
    return f, diff, rep


def compare_backward(orc, x, wl, g, f, diff, grads, tok_mask=None, chunk_mask=None,
                     weights="stick", sel_rows=None):
    """Gradients against the oracle's backward over the GPU's own selection (idx, score, w):
    dQ and dQs on every row of tok_mask, dK, dV and dKslc on every chunk of chunk_mask (default
    all), with no row or chunk left out for a near-tie.  sel_rows [B, L] (optional) limits the
    selection the oracle sees to those rows: valid only when dO is zero on every other row, so
    those rows add exact zeros to every gradient."""
    gi = npy(g["idx"]).astype(np.int32)
    gs, gw = npy(g["score"]), npy(g["w"])
    if sel_rows is not None:
        off = ~np.asarray(sel_rows, bool).reshape(wl.B, wl.L)
        gi, gs, gw = gi.copy(), gs.copy(), gw.copy()
        gi[off], gs[off], gw[off] = -1, -np.inf, 0.0
    o = orc.backward(x["Q"], x["K"], x["V"], x["Qs"], f["Kslc"], gi, gs, gw, x["dO"], wl.S,
                     tok_mask=tok_mask, chunk_mask=chunk_mask, weights=weights)
    tol = tol_for(wl.dtype)
    B, L, nC = wl.B, wl.L, wl.nC
    tm = np.ones((B, L), bool) if tok_mask is None else np.asarray(tok_mask, bool).reshape(B, L)
    cm = np.ones((B, nC), bool) if chunk_mask is None else np.asarray(chunk_mask, bool).reshape(B, nC)
    trow = np.broadcast_to(tm[:, :, None], (B, L, wl.Hkv))
    rep = {}
    rep["dQ"] = max_abs(npy(grads["dQ"]), o["dQ"], head_mask(trow, wl.G))
    rep["dQs"] = max_abs(npy(grads["dQs"]), o["dQs"], trow)
    crow = np.repeat(cm, wl.S, axis=1)  # [B, nC*S]
    crow = np.concatenate([crow, np.zeros((B, L - nC * wl.S), bool)], axis=1)[:, :, None]
    crow = np.broadcast_to(crow, (B, L, wl.Hkv))
    rep["dK"] = max_abs(npy(grads["dK"]), o["dK"], crow)
    rep["dV"] = max_abs(npy(grads["dV"]), o["dV"], crow)
    ck = np.broadcast_to(cm[:, :, None], (B, nC, wl.Hkv))
    rep["dKslc"] = max_abs(npy(grads["dKslc"]), o["dKslc"], ck)
    if chunk_mask is None:  # the incomplete tail chunk's rows must be exactly zero
        assert np.all(npy(grads["dK"])[:, nC * wl.S:] == 0)
        assert np.all(npy(grads["dV"])[:, nC * wl.S:] == 0)
    rep["rows_with_other_selection"] = int(diff.sum())
    say("backward", wl.name, rep)
    for k in ("dQ", "dQs", "dK", "dV", "dKslc"):
        assert rep[k] <= tol, (k, rep[k])
    return rep
