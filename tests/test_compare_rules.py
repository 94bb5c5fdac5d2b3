"""The comparison rules themselves (CPU only): a row whose near-tie is resolved the other way
is accepted as a valid selection, and its outputs and gradients are still checked, against
the oracle over that other selection, so a wrong value there fails.

A stand-in for the GPU library is built from the oracle: the selection of every near-tie
row whose two tied chunks sit in adjacent slots is swapped, the stick-breaking weights are
recomputed for the swapped order, and the outputs and gradients are the oracle's over that
selection rounded to bf16.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from hsa_compare import compare_backward, compare_forward, near_tie_rows

WL = workloads.Workload("cmp_rules", 1, 64 * 7 + 3, 4, 1, 64, 64, 3, torch.bfloat16)


def _inputs():
    x = workloads.make_inputs(WL, seed=41)
    K = x["K"].clone()
    # chunk 1 repeats chunk 0 except one element one bf16 step apart: the two chunk keys
    # differ by about 1e-8, so every row that ranks both has a near-tie between them
    K[:, 64:128] = K[:, 0:64]
    K[0, 64, 0, 0] = torch.tensor(2.0 ** -10, dtype=torch.bfloat16)
    K[0, 0, 0, 0] = torch.tensor(2.0 ** -10 + 2.0 ** -17, dtype=torch.bfloat16)
    x["K"] = K
    return x


def _stick(score):
    w = np.zeros_like(score)
    rem = 1.0
    for k, s in enumerate(score):
        if not np.isfinite(s):
            break
        p = 1.0 / (1.0 + np.exp(-s))
        w[k] = p * rem
        rem *= 1.0 - p
    return w


def _fake_gpu(orc, x):
    Kslc = orc.pool(x["K"], WL.S)
    idx, score, w = orc.select(x["Qs"], Kslc, WL.S, WL.K)
    near = near_tie_rows(orc, x["Qs"], Kslc, WL.S, WL.K)
    swapped = []
    for (b, t, g) in np.argwhere(near):
        row = list(idx[b, t, g])
        if 0 in row and 1 in row and abs(row.index(0) - row.index(1)) == 1:
            i, j = sorted((row.index(0), row.index(1)))
            idx[b, t, g, [i, j]] = idx[b, t, g, [j, i]]
            score[b, t, g, [i, j]] = score[b, t, g, [j, i]]
            w[b, t, g] = _stick(score[b, t, g])
            swapped.append((b, t, g))
    assert len(swapped) >= 5, "the planted near-tie should be resolved the other way somewhere"
    O = orc.attend(x["Q"], x["K"], x["V"], idx, w, WL.S)
    grads = orc.backward(x["Q"], x["K"], x["V"], x["Qs"], Kslc, idx, score, w, x["dO"], WL.S)
    bf = lambda a: torch.from_numpy(np.asarray(a, np.float64)).to(torch.bfloat16)  # noqa: E731
    g = dict(Kslc=bf(Kslc), idx=torch.from_numpy(idx), score=torch.from_numpy(score).float(),
             w=torch.from_numpy(w).float(), O=bf(O))
    gr = {k: bf(grads[k]) for k in ("dQ", "dK", "dV", "dQs")}
    gr["dKslc"] = torch.from_numpy(grads["dKslc"]).float()
    return g, gr, swapped


def test_swapped_near_tie_accepted_and_checked(orc):
    x = _inputs()
    g, gr, swapped = _fake_gpu(orc, x)
    f, diff, rep = compare_forward(orc, x, WL, g)
    assert rep["differing_rows"] == len(swapped)
    compare_backward(orc, x, WL, g, f, diff, gr)
    # a wrong output on a swapped row is caught
    b, t, gg = swapped[len(swapped) // 2]
    bad = dict(g)
    bad["O"] = g["O"].clone()
    bad["O"][b, t, gg * WL.G] += 0.25
    with pytest.raises(AssertionError):
        compare_forward(orc, x, WL, bad)
    # a wrong key gradient in a chunk only the swapped rows changed is caught
    badg = dict(gr)
    badg["dK"] = gr["dK"].clone()
    badg["dK"][b, 64 + 5, gg] += 0.25
    with pytest.raises(AssertionError):
        compare_backward(orc, x, WL, g, f, diff, badg)
    badq = dict(gr)
    badq["dQ"] = gr["dQ"].clone()
    badq["dQ"][b, t, gg * WL.G] += 0.25
    with pytest.raises(AssertionError):
        compare_backward(orc, x, WL, g, f, diff, badq)
