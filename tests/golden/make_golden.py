"""Writes tests/golden/tiny_regression.json from the CPU oracle alone (no GPU code is
imported).  The file pins the oracle against accidental drift; rerun only when a change to
the oracle's arithmetic is justified by a passage of the pages, and say which in the commit.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    wl = workloads.Workload("golden_tiny", 1, 160, 4, 2, 8, 16, 3, workloads.torch.float32,
                            1.0, 1.0)
    x = workloads.make_inputs(wl, seed=123)
    orc = oracle.get()
    f = orc.forward(x["Q"], x["K"], x["V"], x["Qs"], wl.S, wl.K)
    g = orc.backward(x["Q"], x["K"], x["V"], x["Qs"], f["Kslc"], f["idx"], f["score"], f["w"],
                     x["dO"], wl.S)
    rows = [20, 47, 100, 159]
    out = {
        "_about": "oracle output on a seeded tiny case (workloads.make_inputs seed 123); "
                  "written by tests/golden/make_golden.py",
        "shape": dict(B=wl.B, L=wl.L, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, S=wl.S, K=wl.K),
        "rows": rows,
        "idx": f["idx"][0, rows].tolist(),
        "w": f["w"][0, rows].tolist(),
        "O": f["O"][0, rows].tolist(),
        "dQ": g["dQ"][0, rows].tolist(),
        "dK_chunk2": g["dK"][0, 32:48].tolist(),
        "dV_chunk2": g["dV"][0, 32:48].tolist(),
        "dQs": g["dQs"][0, rows].tolist(),
    }
    with open(os.path.join(HERE, "tiny_regression.json"), "w") as fh:
        json.dump(out, fh, indent=1)


if __name__ == "__main__":
    main()
