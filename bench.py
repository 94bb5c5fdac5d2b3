#!/usr/bin/env python3
"""Throughput of the HSA operator on one MI355X, one JSON line on stdout.

A step is one pass of the whole hot path over one batch of synthetic input: hsa_select
(chunk-key pooling, top-K selection, stick-breaking weights), hsa_fwd (softmax-off-by-one
attention inside the selected chunks fused with the weights) and hsa_bwd (two-phase backward
through attention, weights and selection scores), on the fwd_16k workload
(B=4, L=16384, Hq=16, Hkv=2, d=64, S=64, K=8, bf16).  Inputs are resident in HBM before the
timed region starts.  value = B*L tokens per step / seconds per step.

    python bench.py [--steps 20] [--warmup 3] [--no-cpu-baseline] [--decode]

The roofline object describes the entry point that takes the most time; its duration is the
average over the timed steps measured with HIP events on the stream the kernels run on.
cpu_baseline times the CPU oracle (test infrastructure) on a bounded sample of the same
workload; it is a reported baseline, not the target.
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HSA fwd+bwd tokens/sec at L=16K/64K bf16; % HBM roofline / MFMA util"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "chunk_sparse_attention_amd", "csrc", "*"))):
        with open(p, "rb") as fh:
            h.update(os.path.basename(p).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def causal_candidates(wl) -> int:
    per_seq = sum(min(t // wl.S, wl.nC) for t in range(wl.L))
    return wl.B * wl.Hkv * per_seq


def alg_counts(wl, n_slots: int) -> dict:
    """Algorithmic bytes (every input read once, every output written once) and flops per
    launch of each entry point.  n_slots = valid (b, t, g, k) selections."""
    el = 2 if str(wl.dtype).endswith("bfloat16") else 4
    B, L, Hq, Hkv, D, K, S = wl.B, wl.L, wl.Hq, wl.Hkv, wl.D, wl.K, wl.S
    q = B * L * Hq * D * el
    kv = B * L * Hkv * D * el
    kslc = B * wl.nC * Hkv * D * el
    slot = B * L * Hkv * K * 4
    edges_heads = n_slots * wl.G
    return {
        "hsa_select": dict(bytes=2 * kv + kslc + 3 * slot, flops=2 * D * causal_candidates(wl)),
        "hsa_fwd": dict(bytes=q + 2 * kv + 2 * slot + q, flops=4 * S * D * edges_heads),
        "hsa_bwd": dict(bytes=(2 * q + 3 * kv + kslc + 3 * slot) + (q + 3 * kv)
                        + B * wl.nC * Hkv * D * 4,
                        flops=10 * S * D * edges_heads),
    }


def roofline(name: str, counts: dict, avg_ms: float, traffic) -> dict:
    t_hbm = counts["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = counts["flops"] / (BF16_PEAK_TFLOPS * 1e12)
    s = avg_ms / 1e3
    if t_mfma >= t_hbm:
        ach = counts["flops"] / s / 1e12
        r = dict(bound="mfma", achieved=round(ach, 3), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s")
    else:
        ach = counts["bytes"] / s / 1e9
        r = dict(bound="hbm", achieved=round(ach, 2), peak=HBM_PEAK_GBS, unit="GB/s")
    r["frac"] = round(r["achieved"] / r["peak"], 5)
    r["traffic"] = traffic
    r["kernel"] = name
    r["avg_ms"] = round(avg_ms, 4)
    r["alg_bytes"] = int(counts["bytes"])
    r["alg_flops"] = int(counts["flops"])
    return r


def measured_traffic(entry: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{entry}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_sha") != source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(wl, x) -> dict:
    """The oracle (pool, select, attend, backward) on sequence 0 of the workload."""
    import oracle
    orc = oracle.get()
    sl = {k: x[k][:1] for k in ("Q", "K", "V", "Qs", "dO")}
    t0 = time.perf_counter()
    f = orc.forward(sl["Q"], sl["K"], sl["V"], sl["Qs"], wl.S, wl.K)
    orc.backward(sl["Q"], sl["K"], sl["V"], sl["Qs"], f["Kslc"], f["idx"], f["score"], f["w"],
                 sl["dO"], wl.S)
    el = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return dict(value=round(wl.L / el, 2), unit="tokens/s", cores=cores, kind="oracle",
                sample=f"sequence 0 of {wl.B} ({wl.L} tokens): pool+select+attend+backward, "
                       f"{el:.1f} s")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="fwd_16k")
    ap.add_argument("--generic", action="store_true", help="force the vector-ALU kernels")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--decode", action="store_true", help="also time the 1M-context decode step")
    ap.add_argument("--only", choices=["select", "fwd", "bwd"], default=None,
                    help="profiling aid: after one full step, run only this entry point "
                         "--steps times and print its mean time (no JSON line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build of the HSA operator has no multi-GPU "
              f"path (asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import chunk_sparse_attention_amd as hsa
    from chunk_sparse_attention_amd import _lib
    import workloads

    wl = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    log(f"bench: generating {wl.name} inputs")
    x = workloads.make_inputs(wl, seed=0)
    Q, K, V, Qs, dO = (x[k].to(dev) for k in ("Q", "K", "V", "Qs", "dO"))
    prob_bwd = hsa.problem(wl.B, wl.L, wl.Hq, wl.Hkv, wl.D, wl.K, wl.dtype)
    ws_bwd = hsa.workspace(_lib.HSA_OP_BWD, prob_bwd, dev)
    gen = args.generic

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        Kslc, idx, score, w = hsa.select(Qs, K, wl.K, generic=gen)
        if ev is not None:
            ev[1].record()
        O = hsa.fwd(Q, K, V, idx, w, generic=gen)
        if ev is not None:
            ev[2].record()
        g = hsa.bwd(Q, K, V, Qs, Kslc, idx, score, w, dO, generic=gen, ws=ws_bwd)
        if ev is not None:
            ev[3].record()
        return idx, O, g

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        idx, _, _ = step()
    torch.cuda.synchronize()
    n_slots = int((idx >= 0).sum().item())

    if args.only:
        Kslc, idx, score, w = hsa.select(Qs, K, wl.K, generic=gen)
        prob_fwd = hsa.problem(wl.B, wl.L, wl.Hq, wl.Hkv, wl.D, wl.K, wl.dtype, generic=gen)
        ws_fwd = hsa.workspace(_lib.HSA_OP_FWD, prob_fwd, dev)
        O = torch.empty_like(Q)
        run = {"select": lambda: hsa.select(Qs, K, wl.K, generic=gen),
               "fwd": lambda: hsa.fwd(Q, K, V, idx, w, generic=gen, ws=ws_fwd, out=O),
               "bwd": lambda: hsa.bwd(Q, K, V, Qs, Kslc, idx, score, w, dO, generic=gen,
                                      ws=ws_bwd)}[args.only]
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        log(f"bench: only {args.only}: {e0.elapsed_time(e1) / args.steps:.4f} ms per call")
        return 0

    log(f"bench: timing {args.steps} steps")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    names = ["hsa_select", "hsa_fwd", "hsa_bwd"]
    avg = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps
           for j, n in enumerate(names)}
    log("bench: per-entry ms", {k: round(v, 4) for k, v in avg.items()})
    counts = alg_counts(wl, n_slots)
    dominant = max(avg, key=avg.get)
    roof = roofline(dominant, counts[dominant], avg[dominant], measured_traffic(dominant))
    others = {n: roofline(n, counts[n], avg[n], measured_traffic(n)) for n in names}

    tokens = wl.B * wl.L
    out = {
        "metric": METRIC,
        "value": round(tokens / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape; no dataset)",
        "config": {"workload": f"{wl.name}: select+fwd+bwd B={wl.B} L={wl.L} Hq={wl.Hq} "
                               f"Hkv={wl.Hkv} d={wl.D} S={wl.S} K={wl.K}",
                   "global_batch": wl.B, "seq_len": wl.L, "parallelism": "single GPU",
                   "kernels": "generic" if gen else "default"},
        "roofline": roof,
        "entry_points": others,
    }

    if not args.no_secondary:
        wl2 = workloads.WORKLOADS["fwd_64k"]
        log(f"bench: secondary {wl2.name} select+fwd")
        x2 = workloads.make_inputs(wl2, seed=0, with_grad=False)
        Q2, K2, V2, Qs2 = (x2[k].to(dev) for k in ("Q", "K", "V", "Qs"))
        for _ in range(2):
            _, i2, _, w2 = hsa.select(Qs2, K2, wl2.K, generic=gen)
            hsa.fwd(Q2, K2, V2, i2, w2, generic=gen)
        torch.cuda.synchronize()
        n2 = int((i2 >= 0).sum().item())
        reps = max(3, args.steps // 4)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ts, tf = 0.0, 0.0
        for _ in range(reps):
            e[0].record()
            _, i2, _, w2 = hsa.select(Qs2, K2, wl2.K, generic=gen)
            e[1].record()
            hsa.fwd(Q2, K2, V2, i2, w2, generic=gen)
            e[2].record()
            torch.cuda.synchronize()
            ts += e[0].elapsed_time(e[1])
            tf += e[1].elapsed_time(e[2])
        ts /= reps
        tf /= reps
        c2 = alg_counts(wl2, n2)
        out["secondary"] = {
            "workload": f"{wl2.name}: select+fwd B={wl2.B} L={wl2.L} d={wl2.D} K={wl2.K}",
            "select_ms": round(ts, 4), "fwd_ms": round(tf, 4),
            "tokens_per_s": round(wl2.B * wl2.L / ((ts + tf) / 1e3), 1),
            "fwd_roofline": roofline("hsa_fwd", c2["hsa_fwd"], tf, None),
        }
        del Q2, K2, V2, Qs2, x2

    if args.decode:
        wl3 = workloads.WORKLOADS["decode_1m"]
        log(f"bench: decode {wl3.name} (generating caches)")
        x3 = workloads.make_decode_inputs(wl3, seed=0)
        q, qs = x3["q"].to(dev), x3["qs"].to(dev)
        Kc, Vc = x3["Kc"].to(dev), x3["Vc"].to(dev)
        Kslc3 = hsa.pool(Kc)
        prob3 = hsa.problem(wl3.B, wl3.L, wl3.Hq, wl3.Hkv, wl3.D, wl3.K, wl3.dtype)
        ws3 = hsa.workspace(_lib.HSA_OP_DECODE, prob3, dev)
        for _ in range(3):
            hsa.decode(q, qs, Kc, Vc, Kslc3, wl3.K, generic=gen, ws=ws3)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 50
        e0.record()
        for _ in range(reps):
            hsa.decode(q, qs, Kc, Vc, Kslc3, wl3.K, generic=gen, ws=ws3)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / reps
        el = 2
        dbytes = (wl3.B * wl3.nC * wl3.Hkv * wl3.D * el
                  + 2 * wl3.B * wl3.Hkv * wl3.K * wl3.S * wl3.D * el
                  + 2 * wl3.B * wl3.Hq * wl3.D * el + wl3.B * wl3.Hkv * wl3.D * el)
        out["decode"] = {"workload": f"{wl3.name}: B={wl3.B} ctx={wl3.L} K={wl3.K} (warm)",
                         "ms": round(dms, 4), "new_tokens_per_s": round(wl3.B / (dms / 1e3), 1),
                         "hbm_frac": round(dbytes / (dms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}

    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(wl, x)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
