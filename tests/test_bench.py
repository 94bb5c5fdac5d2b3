"""Host-side logic of bench.py (CPU only): the algorithmic counts the roofline is priced
with, the roofline arithmetic and the one-GPU refusal."""
import os
import subprocess
import sys

import pytest
import torch

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_causal_candidates_brute_force():
    """The number of (b, t, g, c) candidates with c < min(floor(t/S), nC), by brute force."""
    wl = workloads.Workload("tiny", 2, 64 * 5 + 17, 4, 3, 64, 64, 4, torch.bfloat16)
    n = 0
    for b in range(wl.B):
        for t in range(wl.L):
            for g in range(wl.Hkv):
                n += sum(1 for c in range(wl.nC) if c < t // wl.S)
    assert bench.causal_candidates(wl) == n


def test_kernel_counts_follow_the_per_unit_figures():
    """Algorithmic bytes and flops per launch: 4 S d flops per (token, head, slot) for the
    forward, 10 S d for the backward's chunk phase, 2 d per causal candidate for selection,
    (S + 1) d element reads and writes per chunk key for pooling."""
    wl = workloads.WORKLOADS["fwd_16k"]
    n_slots = 1_030_144
    c = bench.kernel_counts(wl, n_slots, fused=True, chunked=True)
    eg = n_slots * wl.G
    assert c["fwd"]["flops"] == 4 * wl.S * wl.D * eg
    assert c["bwd_p2"]["flops"] == 10 * wl.S * wl.D * eg
    assert c["select"]["flops"] == 2 * wl.D * bench.causal_candidates(wl)
    # bf16 selection scores on the matrix cores; fp32 selection on the fp64 vector units
    assert not c["select"]["alu"]
    assert bench.kernel_counts(wl, n_slots, mfma_select=False)["select"]["alu"]
    kv = wl.B * wl.L * wl.Hkv * wl.D * 2
    kslc = wl.B * wl.nC * wl.Hkv * wl.D * 2
    assert c["pool"]["bytes"] == kv + kslc
    q = wl.B * wl.L * wl.Hq * wl.D * 2
    slot = wl.B * wl.L * wl.Hkv * wl.K * 4
    # chunk-major forward: Q, K, V and the slots in; the token phase writes O
    assert c["fwd"]["bytes"] == q + 2 * kv + 2 * slot
    assert c["fwd_token"]["bytes"] == q + slot
    # one exponential per logit: S per (token, head, slot), again in the backward's recompute
    assert c["fwd"]["exps"] == c["bwd_p2"]["exps"] == wl.S * eg
    assert "exps" not in c["bwd_p1"]
    r = bench.roofline("fwd", c["fwd"], 0.5, None)
    assert r["exp_floor_ms"] == pytest.approx(wl.S * eg / bench.EXP_PEAK_PER_S * 1e3, abs=1e-4)


def test_roofline_picks_the_binding_peak():
    """A kernel is priced against whichever of HBM and the matrix cores (or the fp64 vector
    units, for ALU-bound selection) its algorithmic counts make the longer."""
    # 8 GB at 8 TB/s = 1 ms beats 1 TFLOP at 2.5 PFLOP/s = 0.4 ms: HBM-bound
    r = bench.roofline("x", dict(bytes=8e9, flops=1e12), 2.0, None)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["amplification"] is None
    assert r["achieved"] == pytest.approx(4000.0) and r["frac"] == pytest.approx(0.5)
    # 1 GB (0.125 ms) against 5 TFLOP (2 ms): MFMA-bound
    r = bench.roofline("y", dict(bytes=1e9, flops=5e12), 4.0, 2.5e9)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["traffic"] == 2.5e9
    assert r["amplification"] == pytest.approx(2.5)  # measured over algorithmic bytes
    assert r["achieved"] == pytest.approx(1250.0) and r["frac"] == pytest.approx(0.5)
    r = bench.roofline("z", dict(bytes=1e6, flops=78.6e9, alu=True), 2.0, None)
    assert r["bound"] == "alu" and r["peak"] == 78.6 and r["frac"] == pytest.approx(0.5)


def test_more_than_one_gpu_is_refused():
    """bench.py --gpus N with N > 1 exits with a message and status 2 (no GPU is touched)."""
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU only" in p.stderr and p.stdout == ""
