"""The oracle against the stored fixtures in tests/golden (closed forms derived from the
pages' definitions, and a regression file written by tests/golden/make_golden.py from the
oracle alone).  CPU only."""
import json
import os

import numpy as np
import torch

import workloads

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


def test_closed_forms(orc):
    cf = _load("closed_forms.json")
    e = cf["equal_scores_weights"]
    S, K = 4, e["K"]
    L = (K + 2) * S
    Km = torch.randn((1, L, 1, 8), generator=torch.Generator().manual_seed(0))
    idx, score, w = orc.select(torch.zeros((1, L, 1, 8)), orc.pool(Km, S), S, K)
    assert list(idx[0, -1, 0]) == e["idx"]
    assert np.array_equal(w[0, -1, 0], np.array(e["w"]))
    assert w[0, -1, 0].sum() == e["sum_w"]

    z = cf["zero_query_probability"]
    S = z["S"]
    L = 2 * S
    V = torch.randn((1, L, 1, 8), generator=torch.Generator().manual_seed(1), dtype=torch.float64)
    idx = torch.full((1, L, 1, 1), -1, dtype=torch.int32)
    idx[0, S:] = 0
    out = orc.attend(torch.zeros((1, L, 1, 8), dtype=torch.float64), torch.zeros_like(V), V,
                     idx, (idx >= 0).double(), S)
    assert np.allclose(out[0, S, 0], z["chunk_output_factor"] * V[0, :S, 0].mean(0).numpy(),
                       rtol=1e-14, atol=0)

    c = cf["causal_slot_counts"]
    S, K = c["S"], c["K"]
    L = max(c["t"]) + 1
    g = torch.Generator().manual_seed(2)
    idx, _, _ = orc.select(torch.randn((1, L, 1, 8), generator=g),
                           orc.pool(torch.randn((1, L, 1, 8), generator=g), S), S, K)
    for t, n in zip(c["t"], c["n_valid"]):
        assert int((idx[0, t, 0] >= 0).sum()) == n, t


def test_tiny_regression(orc):
    gd = _load("tiny_regression.json")
    sh = gd["shape"]
    wl = workloads.Workload("golden_tiny", sh["B"], sh["L"], sh["Hq"], sh["Hkv"], sh["D"],
                            sh["S"], sh["K"], torch.float32, 1.0, 1.0)
    x = workloads.make_inputs(wl, seed=123)
    f = orc.forward(x["Q"], x["K"], x["V"], x["Qs"], wl.S, wl.K)
    g = orc.backward(x["Q"], x["K"], x["V"], x["Qs"], f["Kslc"], f["idx"], f["score"], f["w"],
                     x["dO"], wl.S)
    rows = gd["rows"]
    assert f["idx"][0, rows].tolist() == gd["idx"]
    for key, got in (("w", f["w"][0, rows]), ("O", f["O"][0, rows]), ("dQ", g["dQ"][0, rows]),
                     ("dK_chunk2", g["dK"][0, 32:48]), ("dV_chunk2", g["dV"][0, 32:48]),
                     ("dQs", g["dQs"][0, rows])):
        assert np.allclose(got, np.array(gd[key]), rtol=1e-12, atol=1e-14), key
