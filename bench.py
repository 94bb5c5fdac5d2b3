#!/usr/bin/env python3
"""Throughput of the HSA operator on one MI355X, one JSON line on stdout.

A step is one pass of the whole hot path over one batch of synthetic input: hsa_select
(chunk-key pooling, top-K selection, stick-breaking weights), hsa_fwd (softmax-off-by-one
attention inside the selected chunks fused with the weights) and hsa_bwd (two-phase backward
through attention, weights and selection scores), on the fwd_16k workload
(B=4, L=16384, Hq=16, Hkv=2, d=64, S=64, K=8, bf16).  Inputs are resident in HBM before the
timed region starts.  value = B*L tokens per step / seconds per step.

    python bench.py [--steps 20] [--warmup 3] [--no-cpu-baseline] [--no-secondary]
                    [--no-decode]

The roofline object describes the kernel that takes the most time per step.  Its duration is
the average launch time over a second pass of as many steps, run after the timed ones, from
the HIP events libhsa.so records around each of its launches on the launch's own stream
(hsa_timer_enable / hsa_timer_read); its
algorithmic bytes and flops per launch are the workload's, from kernel_counts().  "kernels"
holds the same for every kernel class, "softmax_weights" the step with the softmax chunk
weights (HSA_FLAG_SOFTMAX_WEIGHTS), "secondary" the select+fwd+bwd pass of the L=65536,
d=128 workload (tokens/s of the whole pass and of select+fwd), "backward_b2" the same pass of
the B=2, L=16384, d=64 backward workload (its hsa_bwd time and tokens/s), "decode" the
1M-context decode step.  cpu_baseline times the CPU oracle (test
infrastructure) on the same workload; it is a reported baseline, not the target.
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HSA fwd+bwd tokens/sec at L=16K/64K bf16; % HBM roofline / MFMA util"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP64_VALU_PEAK_TFLOPS = 78.6   # 256 CUs x 4 SIMD x 16 lanes x 2 (FMA) x 2.4 GHz
# v_exp_f32 results per second: the transcendental unit takes a quarter of the fp32 lane
# rate, 256 CUs x 4 SIMDs x 32 fp32 lanes per clock / 4 x 2.4 GHz (the fp32 vector peak,
# 157.3 TFLOP/s, is the same 32 lanes x 2 flops); the attention's exponentials are priced
# against it as a third floor beside HBM and MFMA
EXP_PEAK_PER_S = 256 * 4 * 32 / 4 * 2.4e9


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


def fused_backward(wl, generic: bool) -> bool:
    """The library's bf16 matrix-core backward: chunk phase with per-edge dQ partials, then a
    token phase."""
    return (not generic and str(wl.dtype).endswith("bfloat16") and wl.D in (64, 128)
            and wl.G in (4, 8, 16) and wl.nC < 32768)


def mfma_select(wl, generic: bool) -> bool:
    """The library's bf16 selection: matrix-core scores of every candidate, fp64 rescoring."""
    return not generic and str(wl.dtype).endswith("bfloat16")


def chunked_forward(wl, generic: bool) -> bool:
    """The library's bf16 chunk-major forward (inverse index, per-edge partials, token sums)."""
    return (not generic and str(wl.dtype).endswith("bfloat16") and wl.D in (64, 128)
            and wl.G in (4, 8, 16) and wl.nC <= 16384)


def kernel_counts(wl, n_slots: int, fused: bool = True, chunked: bool = True,
                  mfma_select: bool = True) -> dict:
    """Algorithmic bytes (each input the kernel needs read once, each output it produces
    written once; workspace copies of the design are not counted) and flops per launch of
    each kernel class.  n_slots = valid (b, t, g, k) selections; every slot is attended by
    G query heads over S keys.  Selection scores every candidate on the matrix cores when
    mfma_select (bf16: the products are exact there, and only about K candidates per token
    are rescored in fp64), else on the fp64 vector units.  "exps" counts the exponentials: one per logit in the forward
    and one per logit again where the backward recomputes the probabilities."""
    el = 2 if str(wl.dtype).endswith("bfloat16") else 4
    B, L, Hq, Hkv, D, K, S = wl.B, wl.L, wl.Hq, wl.Hkv, wl.D, wl.K, wl.S
    q = B * L * Hq * D * el                 # Q, dO, O or dQ
    kv = B * L * Hkv * D * el               # K, V, Qs, dQs, dK or dV
    kslc = B * wl.nC * Hkv * D * el         # Kslc
    slot = B * L * Hkv * K * 4              # idx, score, w or ds
    eg = n_slots * wl.G
    c = {
        "pool": dict(bytes=kv + kslc, flops=B * wl.nC * Hkv * D * S),
        "select": dict(bytes=kv + kslc + 3 * slot, flops=2 * D * causal_candidates(wl),
                       alu=not mfma_select),
        "tile_prep": dict(bytes=slot, flops=0),
        "prep_ops": dict(bytes=2 * kv, flops=0),
        "fwd": dict(bytes=2 * q + 2 * kv + 2 * slot, flops=4 * S * D * eg, exps=S * eg),
        "invidx": dict(bytes=slot + 4 * n_slots, flops=0),
        "bwd_p1": dict(bytes=3 * q + 4 * kv + kslc + 4 * slot, flops=6 * S * D * eg,
                       exps=S * eg),
        "bwd_p2": dict(bytes=2 * q + 5 * kv + 2 * slot + 4 * n_slots + 2 * kslc,
                       flops=8 * S * D * eg, exps=S * eg),
        "bwd_reduce": dict(bytes=2 * kv + 2 * kslc, flops=0),
    }
    if chunked:
        # chunk-major forward: Q, K, V and the slots in (the token phase writes O)
        c["fwd"] = dict(bytes=q + 2 * kv + 2 * slot, flops=4 * S * D * eg, exps=S * eg)
        c["fwd_token"] = dict(bytes=q + slot, flops=0)
    if fused:
        # token phase: dQ and dQs out, the slots and Kslc rows in; dKslc partials read Qs
        c["bwd_p1"] = dict(bytes=q + 2 * kv + kslc + 3 * slot, flops=0)
        # chunk phase: Q, dO, K, V and the weights in; S, dP, dV, dK and dQ products
        c["bwd_p2"] = dict(bytes=2 * q + 2 * kv + slot, flops=10 * S * D * eg, exps=S * eg)
    return c


def roofline(name: str, counts: dict, avg_ms: float, traffic) -> dict:
    """Price one kernel's average launch against MI355X's peaks: HBM bandwidth, dense bf16
    MFMA or, for scoring on the fp64 vector units, the fp64 vector rate."""
    t_hbm = counts["bytes"] / (HBM_PEAK_GBS * 1e9)
    alu = counts.get("alu", False)
    peak_f = FP64_VALU_PEAK_TFLOPS if alu else BF16_PEAK_TFLOPS
    t_f = counts["flops"] / (peak_f * 1e12)
    s = avg_ms / 1e3
    if t_f >= t_hbm:
        ach = counts["flops"] / s / 1e12
        r = dict(bound="alu" if alu else "mfma", achieved=round(ach, 3), peak=peak_f,
                 unit="TFLOP/s")
    else:
        ach = counts["bytes"] / s / 1e9
        r = dict(bound="hbm", achieved=round(ach, 2), peak=HBM_PEAK_GBS, unit="GB/s")
    r["frac"] = round(r["achieved"] / r["peak"], 5)
    r["traffic"] = traffic
    # measured HBM bytes over the algorithmic bytes (re-reads and the design's workspace)
    r["amplification"] = (round(traffic / counts["bytes"], 2)
                          if traffic is not None and counts["bytes"] else None)
    r["kernel"] = name
    r["avg_ms"] = round(avg_ms, 4)
    r["alg_bytes"] = int(counts["bytes"])
    r["alg_flops"] = int(counts["flops"])
    if counts.get("exps"):
        r["exps"] = int(counts["exps"])
        r["exp_floor_ms"] = round(counts["exps"] / EXP_PEAK_PER_S * 1e3, 4)
    return r


# kernel function name -> kernel class of the launch timer; the first matching prefix wins.
# A class launch is one host call: the inverse index runs four kernels per launch and the
# fused backward's token phase two; the others are one kernel each.
KERNEL_CLASS_OF = (("k_bwd_p2_reduce", "bwd_reduce"), ("k_bwd_p2", "bwd_p2"),
                   ("k_bwd_chunk", "bwd_p2"), ("k_bwd_p1", "bwd_p1"), ("k_bwd_tok", "bwd_p1"),
                   ("k_bwd_dks", "bwd_p1"), ("k_inv_", "invidx"), ("k_tile_prep", "tile_prep"),
                   ("k_prep_ops", "prep_ops"), ("k_fwd_tok", "fwd_token"), ("k_fwd_", "fwd"),
                   ("k_select", "select"),
                   ("k_pool", "pool"), ("k_dec_scan", "decode_scan"),
                   ("k_dec_attend", "decode_attend"))
# kernels that run inside another kernel's class launch (not counted as launches)
SECONDARY_KERNELS = {"k_inv_count", "k_inv_colscan", "k_inv_scan", "k_bwd_dks"}


def kernel_class(kernel_name: str):
    m = re.search(r"hsa::(k_[a-z0-9_]+)", kernel_name)
    if not m:
        return None, None
    for prefix, cls in KERNEL_CLASS_OF:
        if m.group(1).startswith(prefix):
            return cls, m.group(1)
    return None, m.group(1)


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def measured_traffic(workload: str, cls: str):
    """HBM bytes per launch of one kernel class, from the committed rocprofv3 counter summary
    of the workload, if it was taken on the current kernel sources; otherwise None."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_sha") != source_sha():
        return None
    k = t.get("kernels", {}).get(cls)
    return None if k is None else k["hbm_bytes_per_launch"]


def decode_traffic():
    """Measured HBM bytes of one decode_1m step (scan + attend), from the committed counter
    summary of `bench.py --only decode_step`, if taken on the current sources."""
    a = measured_traffic("decode_1m", "decode_scan")
    b = measured_traffic("decode_1m", "decode_attend")
    return None if a is None or b is None else a + b


def summarize_counters(cdir: str, workload: str, copy_mib: int) -> int:
    """Turn two rocprofv3 --pmc runs of `bench.py --only step --copy-mib M` (FETCH_SIZE under
    cdir/fetch, WRITE_SIZE under cdir/write) into HBM bytes per launch of each kernel class.
    Each counter is scaled by what it reads for the plain device copy of M MiB that the run
    makes first (a copy reads M MiB and writes M MiB).  Writes profiles/traffic_<workload>.json
    and prints a markdown table."""
    import collections
    import csv
    vals = {}
    for sub, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        files = glob.glob(os.path.join(cdir, sub, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            log(f"bench: no counter_collection.csv under {cdir}/{sub}")
            return 1
        per = collections.defaultdict(list)
        with open(files[0]) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    per[r["Kernel_Name"]].append(float(r["Counter_Value"]) * 1024.0)
        vals[counter] = per
    copies = [(max(v), k) for k, v in vals["FETCH_SIZE"].items() if "copy" in k.lower()]
    if not copies:
        log("bench: no copy kernel in the FETCH_SIZE run")
        return 1
    cf, ck = max(copies)
    cw = max(vals["WRITE_SIZE"][ck])
    ref = copy_mib * 2.0 ** 20
    fs, wsc = ref / cf, ref / cw
    acc = collections.defaultdict(lambda: dict(fetch=0.0, write=0.0, launches=0, names=set()))
    for name, fv in vals["FETCH_SIZE"].items():
        cls, fn = kernel_class(name)
        if cls is None:
            continue
        a = acc[cls]
        a["fetch"] += sum(fv) * fs
        a["write"] += sum(vals["WRITE_SIZE"].get(name, [])) * wsc
        if fn not in SECONDARY_KERNELS:
            a["launches"] += len(fv)
        a["names"].add(re.sub(r"\(.*", "", name).replace("void ", "").strip())
    out = {"source_sha": source_sha(), "workload": workload,
           "copy_reference": {"mib": copy_mib, "kernel": re.sub(r"\(.*", "", ck)[:100],
                              "fetch_read_over_true": round(cf / ref, 4),
                              "write_read_over_true": round(cw / ref, 4)},
           "kernels": {}}
    print(f"| kernel class | launches | FETCH MB/launch | WRITE MB/launch | HBM MB/launch | kernels |")
    print("|---|---:|---:|---:|---:|---|")
    for cls in sorted(acc, key=lambda c: -(acc[c]["fetch"] + acc[c]["write"])):
        a = acc[cls]
        n = max(a["launches"], 1)
        f, w = a["fetch"] / n, a["write"] / n
        out["kernels"][cls] = dict(launches=a["launches"], fetch_bytes_per_launch=round(f),
                                   write_bytes_per_launch=round(w),
                                   hbm_bytes_per_launch=round(f + w), kernels=sorted(a["names"]))
        print(f"| {cls} | {a['launches']} | {f / 1e6:.1f} | {w / 1e6:.1f} | {(f + w) / 1e6:.1f} "
              f"| {', '.join('`' + k + '`' for k in sorted(a['names']))} |")
    print(f"\nCopy reference ({copy_mib} MiB, `{out['copy_reference']['kernel'][:60]}`): "
          f"FETCH_SIZE reads {cf / ref:.3f} x and WRITE_SIZE {cw / ref:.3f} x the bytes moved; "
          f"the figures above are scaled by {fs:.3f} and {wsc:.3f}.")
    with open(traffic_path(workload), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    # optional runs of the same command with L2 (DIR/l2), SQ (DIR/sq) and matrix-core / LDS
    # (DIR/mx) counters
    extra = collections.defaultdict(lambda: collections.defaultdict(list))
    for sub in ("l2", "sq", "mx"):
        for f in glob.glob(os.path.join(cdir, sub, "**", "*counter_collection.csv"),
                           recursive=True)[:1]:
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    cls, fn = kernel_class(r["Kernel_Name"])
                    if cls:
                        extra[fn][r["Counter_Name"]].append(float(r["Counter_Value"]))
    l2sq = {fn: c for fn, c in extra.items() if "TCC_HIT_sum" in c or "SQ_WAVES" in c}
    if l2sq:
        print("\n| kernel | L2 hit rate | waves | per wave: VALU | MFMA | LDS | VMEM rd | "
              "wave cycles | waiting cycles |")
        print("|---|---:|---:|---:|---:|---:|---:|---:|---:|")
        for fn, c in sorted(l2sq.items()):
            m = {k: sum(v) / len(v) for k, v in c.items()}
            hit = m.get("TCC_HIT_sum", 0.0)
            tot = hit + m.get("TCC_MISS_sum", 0.0)
            wv = m.get("SQ_WAVES", 0.0)

            def pw(k):
                return f"{m[k] / wv:.0f}" if wv and k in m else "-"
            print(f"| `{fn}` | {hit / tot:.3f} | {wv:.0f} | {pw('SQ_INSTS_VALU')} | "
                  f"{pw('SQ_INSTS_MFMA')} | {pw('SQ_INSTS_LDS')} | {pw('SQ_INSTS_VMEM_RD')} | "
                  f"{pw('SQ_WAVE_CYCLES')} | {pw('SQ_WAIT_INST_ANY')} |" if tot else
                  f"| `{fn}` | - | {wv:.0f} | - | - | - | - | - | - |")
    mx = {fn: {k: sum(v) / len(v) for k, v in c.items()} for fn, c in extra.items()
          if "MfmaUtil" in c}
    if mx:
        # rocprofv3's derived metrics: MfmaUtil = matrix-core busy cycles over (GPU active
        # cycles x SIMDs), in %; LdsBankConflict = bank-conflict stall cycles per LDS active
        # cycle that was not a stall; LDSBankConflict = those stalls in % of GPU time.
        # SQ_INSTS_VALU_MFMA_MOPS_BF16 counts executed bf16 matrix flops / 512.
        print("\n| kernel | MFMA busy % | bf16 MFMA GFLOP executed per dispatch | "
              "LDS bank-conflict cycles per access cycle | LDS bank-conflict % of time |")
        print("|---|---:|---:|---:|---:|")
        for fn, m in sorted(mx.items()):
            print(f"| `{fn}` | {m.get('MfmaUtil', 0.0):.1f} | "
                  f"{m.get('SQ_INSTS_VALU_MFMA_MOPS_BF16', 0.0) * 512 / 1e9:.1f} | "
                  f"{m.get('LdsBankConflict', 0.0):.3f} | {m.get('LDSBankConflict', 0.0):.2f} |")
    return 0


def summarize_trace(tdir: str, bench_json: str) -> int:
    """Markdown tables of a rocprofv3 --kernel-trace --stats run under tdir: the per-kernel
    statistics (run_kernel_stats.csv), the same split by launch grid (run_kernel_trace.csv;
    one workload's launches share a grid), and the per-launch averages the bench's own
    HIP-event timer printed beside those of the launch grid with the most calls (the bench
    step's: it runs more steps than any other leg)."""
    import collections
    import csv

    def short(n):
        return re.sub(r"\(.*", "", n).replace("void ", "").strip()

    files = glob.glob(os.path.join(tdir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        log(f"bench: no kernel_stats.csv under {tdir}")
        return 1
    rows = list(csv.DictReader(open(files[0])))
    print("| kernel | calls | avg µs | min µs | max µs | % of GPU time |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows:
        print(f"| `{short(r['Name'])[:90]}` | {int(r['Calls'])} | "
              f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
              f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    tfiles = glob.glob(os.path.join(tdir, "**", "*kernel_trace.csv"), recursive=True)
    shapes = collections.defaultdict(list)
    if tfiles:
        for r in csv.DictReader(open(tfiles[0])):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            shapes[(short(r["Kernel_Name"]), grid)].append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        print("\n| kernel (library kernels) | grid (work-items) | calls | avg µs | min µs | max µs |")
        print("|---|---:|---:|---:|---:|---:|")
        for (name, grid), d in sorted(shapes.items()):
            if kernel_class(name)[0] is None:
                continue
            print(f"| `{name[:90]}` | {grid} | {len(d)} | {sum(d) / len(d):.1f} | "
                  f"{min(d):.1f} | {max(d):.1f} |")
    by_cls = {}
    for (name, grid), d in shapes.items():
        cls, _ = kernel_class(name)
        if cls is None:
            continue
        best = by_cls.setdefault(cls, {})
        if name not in best or len(d) > best[name][0]:
            best[name] = (len(d), grid, sum(d) / len(d))
    with open(bench_json) as fh:
        b = json.loads(fh.read().strip().splitlines()[-1])
    print("\n| kernel class | bench.py avg ms per launch | rocprofv3 avg ms per kernel (grid, calls) |")
    print("|---|---:|---|")
    for cls, k in sorted(b["kernels"].items(), key=lambda kv: -kv[1]["ms_per_step"]):
        cell = "; ".join(f"`{n}` {avg / 1e3:.4f} ({grid}, {c})"
                         for n, (c, grid, avg) in sorted(by_cls.get(cls, {}).items()))
        print(f"| {cls} | {k['avg_ms']:.4f} | {cell} |")
    return 0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads() -> int:
    """Threads the oracle's OpenMP loops use by default: OMP_NUM_THREADS when set, else one
    per CPU of the affinity mask."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    return int(env) if env.isdigit() else len(os.sched_getaffinity(0))


def median_seconds(fn, reps: int = 3) -> float:
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[len(ts) // 2]


def oracle_rates(orc, tokens: int, fn, threads: int) -> dict:
    """Median of three timed runs of fn at `threads` and at one thread; tokens/s of each."""
    out = {}
    for n in (threads, 1):
        orc.set_threads(n)
        sec = median_seconds(fn)
        out["threads_%d" % n] = dict(seconds=round(sec, 3), tokens_per_s=round(tokens / sec, 2))
    orc.set_threads(threads)
    return out


def cpu_baseline(wl, x, wl2, x2, every: int = 8, every2: int = 32) -> dict:
    """The oracle (test infrastructure, untuned) on the host cores, on bounded samples of the
    workloads: median of three runs at all threads and at one thread.
      step (fwd_16k): sequence 0, every `every`-th token: pooling of the whole sequence, then
        selection, attention and the whole backward for the sampled tokens only (the other
        rows select nothing, so both backward phases do the sampled tokens' work);
      select+fwd (fwd_64k): every `every2`-th token, pooling of the whole sequence.
    Per-token work does not depend on the token's position except selection, which grows
    with the number of earlier chunks; every k-th token samples those positions evenly, so
    tokens/s = sampled tokens / seconds is the rate of the whole workload."""
    import numpy as np
    import oracle
    orc = oracle.get()
    threads = cpu_threads()
    sl = {k: x[k][0:1] for k in ("Q", "K", "V", "Qs", "dO")}
    rows = np.zeros((1, wl.L), np.uint8)
    rows[0, ::every] = 1
    n_rows = int(rows.sum())

    def step():
        Kslc = orc.pool(sl["K"], wl.S)
        idx, score, w = orc.select(sl["Qs"], Kslc, wl.S, wl.K, row_mask=rows)
        orc.attend(sl["Q"], sl["K"], sl["V"], idx, w, wl.S, row_mask=rows)
        orc.backward(sl["Q"], sl["K"], sl["V"], sl["Qs"], Kslc, idx, score, w, sl["dO"], wl.S)

    rows2 = np.zeros((wl2.B, wl2.L), np.uint8)
    rows2[:, ::every2] = 1
    n_rows2 = int(rows2.sum())

    def select_fwd():
        Kslc = orc.pool(x2["K"], wl2.S)
        idx, _, w = orc.select(x2["Qs"], Kslc, wl2.S, wl2.K, row_mask=rows2)
        orc.attend(x2["Q"], x2["K"], x2["V"], idx, w, wl2.S, row_mask=rows2)

    r1 = oracle_rates(orc, n_rows, step, threads)
    r2 = oracle_rates(orc, n_rows2, select_fwd, threads)
    head = r1["threads_%d" % threads]
    return dict(value=head["tokens_per_s"], unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{wl.name} step (pool+select+attend+backward), sequence 0, every "
                       f"{every}th token ({n_rows} tokens); median of 3",
                cpu=cpu_model(),
                configs={f"{wl.name}_step": dict(sample=f"sequence 0, every {every}th token",
                                                 **r1),
                         f"{wl2.name}_select_fwd": dict(sample=f"every {every2}th token",
                                                        **r2)})


def run_decode(hsa, _lib, workloads, dev, gen: bool, reps: int, cpu: bool = False) -> dict:
    """Time the 1M-context decode step (decode_1m), caches resident in HBM (back to back, and
    cold: the median step after the last-level cache was flushed), and its variants.  cpu:
    also time the oracle's decode step on the host (median of three, all threads and one
    thread; its chunk-key table is pooled first and not timed, as on the GPU)."""
    import torch
    wl3 = workloads.WORKLOADS["decode_1m"]
    log(f"bench: decode {wl3.name} (generating caches)")
    x3 = workloads.make_decode_inputs(wl3, seed=0, slab=4)
    q, qs = x3["q"].to(dev), x3["qs"].to(dev)
    Kc, Vc = x3["Kc"].to(dev), x3["Vc"].to(dev)
    # the same caches in pinned host memory for the offloaded step
    Kh, Vh = x3["Kc"].pin_memory(), x3["Vc"].pin_memory()
    del x3
    Kslc3 = hsa.pool(Kc)
    prob3 = hsa.problem(wl3.B, wl3.L, wl3.Hq, wl3.Hkv, wl3.D, wl3.K, wl3.dtype, generic=gen)
    ws3 = hsa.workspace(_lib.HSA_OP_DECODE, prob3, dev)
    for _ in range(3):
        hsa.decode(q, qs, Kc, Vc, Kslc3, wl3.K, generic=gen, ws=ws3)
    torch.cuda.synchronize()
    log("bench: decode timing")
    # back-to-back steps without the kernel timer (its event records are not negligible at
    # this scale), then the same with it for the per-kernel split
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        hsa.decode(q, qs, Kc, Vc, Kslc3, wl3.K, generic=gen, ws=ws3)
    e1.record()
    torch.cuda.synchronize()
    dms = e0.elapsed_time(e1) / reps
    # the same step captured in a HIP graph and replayed (decode is launch-bound)
    sd = torch.cuda.Stream()
    sd.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(sd):
        hsa.decode(q, qs, Kc, Vc, Kslc3, wl3.K, generic=gen, ws=ws3)
    torch.cuda.current_stream().wait_stream(sd)
    gdec = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gdec):
        hsa.decode(q, qs, Kc, Vc, Kslc3, wl3.K, generic=gen, ws=ws3)
    gdec.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        gdec.replay()
    e1.record()
    torch.cuda.synchronize()
    gms = e0.elapsed_time(e1) / reps
    del gdec
    # cold: 512 MiB read before every step pushes the chunk-key table out of the 256 MB
    # last-level cache (a read, so that no write-back overlaps the step); only the step
    # itself is timed
    flush = torch.ones(1 << 27, dtype=torch.float32, device=dev)
    cold = []
    for r in range(reps // 2):
        flush.sum()
        e0.record()
        hsa.decode(q, qs, Kc, Vc, Kslc3, wl3.K, generic=gen, ws=ws3)
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush
    cms = sorted(cold)[len(cold) // 2]
    hsa.timer_enable(True)
    for _ in range(reps):
        hsa.decode(q, qs, Kc, Vc, Kslc3, wl3.K, generic=gen, ws=ws3)
    torch.cuda.synchronize()
    hsa.timer_enable(False)
    kt3 = hsa.timer_read()
    n3 = kt3["decode_attend"][0]
    tot3 = kt3["decode_scan"][1] + kt3["decode_attend"][1]
    # the step with the caches left in host memory: only the selected chunks cross the link
    for _ in range(3):
        hsa.decode_host_kv(q, qs, Kh, Vh, Kslc3, wl3.K, generic=gen, ws=ws3)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        hsa.decode_host_kv(q, qs, Kh, Vh, Kslc3, wl3.K, generic=gen, ws=ws3)
    e1.record()
    torch.cuda.synchronize()
    hms = e0.elapsed_time(e1) / reps
    cpu_dec = None
    if cpu:
        import oracle
        orc = oracle.get()
        log("bench: cpu baseline of the decode step (oracle)")
        qh, qsh = q.cpu(), qs.cpu()
        ksh = orc.pool(Kh, wl3.S)
        cpu_dec = dict(sample=f"the whole step, {wl3.B} sequences", cores=cpu_threads(),
                       **oracle_rates(orc, wl3.B, lambda: orc.decode(qh, qsh, Kh, Vh, ksh, wl3.S,
                                                                     wl3.K), cpu_threads()))
        del ksh
    del Kh, Vh
    # sequences of different lengths in the same cache (hsa_decode_ragged): lengths drawn
    # uniformly from [ctx/2, ctx] with a fixed seed
    g = torch.Generator().manual_seed(1)
    lens = torch.randint(wl3.L // 2, wl3.L + 1, (wl3.B,), generator=g, dtype=torch.int32)
    ctx_lens = lens.to(dev)
    for _ in range(3):
        hsa.decode_ragged(q, qs, Kc, Vc, Kslc3, ctx_lens, wl3.K, generic=gen, ws=ws3)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        hsa.decode_ragged(q, qs, Kc, Vc, Kslc3, ctx_lens, wl3.K, generic=gen, ws=ws3)
    e1.record()
    torch.cuda.synchronize()
    rms = e0.elapsed_time(e1) / reps
    del Kc, Vc
    # four layers at a 16K context sharing one selection (hsa_decode for the first layer,
    # hsa_decode_shared for the other three) against four independent decode steps
    nl, ctx4 = 4, 16384
    wl4 = workloads.Workload("decode_16k_layers", wl3.B, ctx4, wl3.Hq, wl3.Hkv, wl3.D, wl3.S,
                             wl3.K, wl3.dtype, decode=True)
    xs = [workloads.make_decode_inputs(wl4, seed=10 + l) for l in range(nl)]
    q4 = torch.stack([x["q"] for x in xs]).to(dev)
    K4 = torch.stack([x["Kc"] for x in xs]).to(dev)
    V4 = torch.stack([x["Vc"] for x in xs]).to(dev)
    qs4 = [x["qs"].to(dev) for x in xs]
    del xs
    ks4 = [hsa.pool(K4[l]) for l in range(nl)]

    def shared():
        _, i4, _, w4 = hsa.decode(q4[0], qs4[0], K4[0], V4[0], ks4[0], wl4.K, generic=gen)
        hsa.decode_shared(q4[1:], K4[1:], V4[1:], i4, w4)

    def unshared():
        for l in range(nl):
            hsa.decode(q4[l], qs4[l], K4[l], V4[l], ks4[l], wl4.K, generic=gen)

    # the same with every layer's caches in pinned host memory
    Kh4, Vh4 = K4.cpu().pin_memory(), V4.cpu().pin_memory()

    def shared_host():
        _, i4, _, w4 = hsa.decode_host_kv(q4[0], qs4[0], Kh4[0], Vh4[0], ks4[0], wl4.K,
                                          generic=gen)
        hsa.decode_shared(q4[1:], Kh4[1:], Vh4[1:], i4, w4)

    def unshared_host():
        for l in range(nl):
            hsa.decode_host_kv(q4[l], qs4[l], Kh4[l], Vh4[l], ks4[l], wl4.K, generic=gen)

    lay = {}
    for name, fn in (("shared_ms", shared), ("unshared_ms", unshared),
                     ("host_kv_shared_ms", shared_host), ("host_kv_unshared_ms", unshared_host)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        lay[name] = round(e0.elapsed_time(e1) / reps, 4)
    del q4, K4, V4, qs4, ks4, Kh4, Vh4
    el = 2
    # the chunk-key table, the selected chunks' K and V, q, qs and O
    dbytes = (wl3.B * wl3.nC * wl3.Hkv * wl3.D * el
              + 2 * wl3.B * wl3.Hkv * wl3.K * wl3.S * wl3.D * el
              + 2 * wl3.B * wl3.Hq * wl3.D * el + wl3.B * wl3.Hkv * wl3.D * el)
    return {"workload": f"{wl3.name}: B={wl3.B} ctx={wl3.L} Hq={wl3.Hq} Hkv={wl3.Hkv} "
                        f"d={wl3.D} K={wl3.K}",
            "ms": round(dms, 4), "new_tokens_per_s": round(wl3.B / (dms / 1e3), 1),
            "cold_ms_median": round(cms, 4), "graph_ms": round(gms, 4),
            "roofline": roofline("decode_scan+decode_attend", dict(bytes=dbytes, flops=0),
                                 tot3 / max(n3, 1), decode_traffic()),
            "scan_ms": round(kt3["decode_scan"][1] / max(n3, 1), 4),
            "attend_ms": round(kt3["decode_attend"][1] / max(n3, 1), 4),
            "host_kv": {"ms": round(hms, 4), "vs_device_kv": round(hms / dms, 3),
                        "link_bytes_per_step": 2 * wl3.B * wl3.Hkv * wl3.K * wl3.S * wl3.D * el},
            "ragged": {"ms": round(rms, 4), "mean_ctx": round(float(lens.double().mean()), 1),
                       "lengths": "uniform in [ctx/2, ctx], seed 1"},
            "shared_selection": {"workload": f"{nl} layers, B={wl4.B} ctx={ctx4} Hq={wl4.Hq} "
                                             f"Hkv={wl4.Hkv} d={wl4.D} K={wl4.K}", **lay},
            "cpu_baseline": cpu_dec}


def run_pass(hsa, _lib, workloads, dev, gen: bool, name: str, reps: int) -> dict:
    """One select+fwd+bwd pass over another workload, timed per entry point with events on the
    current stream and per kernel class with the library's launch timer (average over reps
    passes after two untimed ones)."""
    import torch
    wl2 = workloads.WORKLOADS[name]
    log(f"bench: {wl2.name} select+fwd+bwd")
    x2 = workloads.make_inputs(wl2, seed=0)
    Q2, K2, V2, Qs2, dO2 = (x2[k].to(dev) for k in ("Q", "K", "V", "Qs", "dO"))
    del x2
    prob2 = hsa.problem(wl2.B, wl2.L, wl2.Hq, wl2.Hkv, wl2.D, wl2.K, wl2.dtype, generic=gen)
    ws2 = hsa.workspace(_lib.HSA_OP_BWD, prob2, dev)
    O2 = torch.empty_like(Q2)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def step2():
        Kslc2, i2, sc2, w2 = hsa.select(Qs2, K2, wl2.K, generic=gen)
        e[1].record()
        hsa.fwd(Q2, K2, V2, i2, w2, generic=gen, ws=ws2, out=O2)
        e[2].record()
        hsa.bwd(Q2, K2, V2, Qs2, Kslc2, i2, sc2, w2, dO2, generic=gen, ws=ws2,
                after_fwd=True)
        return i2

    for _ in range(2):
        i2 = step2()
    torch.cuda.synchronize()
    n2 = int((i2 >= 0).sum().item())
    ts, tf, tb = 0.0, 0.0, 0.0
    hsa.timer_enable(True)
    for _ in range(reps):
        e[0].record()
        step2()
        e[3].record()
        torch.cuda.synchronize()
        ts += e[0].elapsed_time(e[1])
        tf += e[1].elapsed_time(e[2])
        tb += e[2].elapsed_time(e[3])
    hsa.timer_enable(False)
    kt2 = hsa.timer_read()
    ts /= reps
    tf /= reps
    tb /= reps
    c2 = kernel_counts(wl2, n2, fused_backward(wl2, gen), chunked_forward(wl2, gen),
                       mfma_select(wl2, gen))
    k2 = {k: roofline(k, c2[k], total / n, measured_traffic(wl2.name, k))
          for k, (n, total) in kt2.items() if n}
    tokens = wl2.B * wl2.L
    r = {
        "workload": f"{wl2.name}: select+fwd+bwd B={wl2.B} L={wl2.L} Hq={wl2.Hq} "
                    f"Hkv={wl2.Hkv} d={wl2.D} K={wl2.K}",
        "select_ms": round(ts, 4), "fwd_ms": round(tf, 4), "bwd_ms": round(tb, 4),
        "tokens_per_s": round(tokens / ((ts + tf + tb) / 1e3), 1),
        "fwd_tokens_per_s": round(tokens / ((ts + tf) / 1e3), 1),
        "bwd_tokens_per_s": round(tokens / (tb / 1e3), 1),
        "kernels": k2,
    }
    del Q2, K2, V2, Qs2, dO2, O2, ws2
    return r


def copy_reference(dev, mib: int) -> None:
    """Profiling aid: one plain device copy of `mib` MiB whose source was first pushed out of
    the 256 MB last-level cache (by writing 1 GiB elsewhere), so the copy reads it from HBM;
    its byte counters scale the counters of the kernels that follow."""
    if not mib:
        return
    import torch
    src = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"bench: copied {mib} MiB")
    del src, dst, flush


def ceilings(dev, reps: int = 20) -> dict:
    """Streaming rates of plain device kernels (torch's own): a read (sum of 2 GiB of fp32), a
    write (fill of 2 GiB) and a copy (1 GiB to 1 GiB), each far larger than the 256 MB
    last-level cache, and a read of 128 MiB that was just written (served by that cache).
    The practical ceilings the kernels' measured traffic is compared with."""
    import torch
    big = torch.ones(1 << 29, dtype=torch.float32, device=dev)   # 2 GiB
    half = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    small = torch.ones(1 << 25, dtype=torch.float32, device=dev)  # 128 MiB
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def rate(fn, nbytes, prep=None):
        for _ in range(2):
            if prep:
                prep()
            fn()
        torch.cuda.synchronize()
        t = 0.0
        for _ in range(reps):
            if prep:
                prep()
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t += e0.elapsed_time(e1)
        return round(nbytes / (t / reps / 1e3) / 1e9, 1)

    # reads: several reductions with small outputs, the best one taken as the read rate
    reads = {"sum": lambda t: t.sum(),
             "row_sums_256": lambda t: t.view(-1, 256).sum(1),
             "row_max_4096": lambda t: t.view(-1, 4096).amax(1),
             "dot": lambda t: torch.dot(t, t)}
    rd = {k: rate(lambda f=f: f(big), big.numel() * 4) for k, f in reads.items()}
    rs = {k: rate(lambda f=f: f(small), small.numel() * 4, prep=lambda: small.fill_(2.0))
          for k, f in reads.items()}
    out = {"read_2GiB_GBs": max(rd.values()), "read_2GiB_by_kernel": rd,
           "write_2GiB_GBs": rate(lambda: big.fill_(1.0), big.numel() * 4),
           "copy_1GiB_GBs": rate(lambda: half.copy_(big[:1 << 28]), 2 * half.numel() * 4),
           "read_128MiB_after_write_GBs": max(rs.values()),
           "read_128MiB_after_write_by_kernel": rs}
    del big, half, small
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="fwd_16k")
    ap.add_argument("--generic", action="store_true", help="force the vector-ALU kernels")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the 1M-context decode step")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the step (an informational figure)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="profiling aid: with --only, first copy this many MiB once with a plain "
                         "device copy (the scale reference for HBM byte counters)")
    ap.add_argument("--ceilings", action="store_true",
                    help="print the streaming rates of plain device kernels (read, write, copy, "
                         "a cache-resident read) as one JSON line and exit")
    ap.add_argument("--only", choices=["step", "select", "fwd", "bwd", "decode", "decode_step"],
                    default=None,
                    help="profiling aid: after the warm-up, run only this entry point (or the "
                         "whole step) --steps times and print its mean time (no JSON line)")
    ap.add_argument("--summarize-counters", metavar="DIR", default=None,
                    help="write profiles/traffic_<workload>.json from the FETCH_SIZE (DIR/fetch) "
                         "and WRITE_SIZE (DIR/write) runs of --only step --copy-mib M; no GPU")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "BENCH_JSON"), default=None,
                    help="markdown table of a --kernel-trace --stats run beside the bench's "
                         "own per-launch timing; no GPU")
    args = ap.parse_args()
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters, args.workload, args.copy_mib)
    if args.summarize_trace:
        return summarize_trace(*args.summarize_trace)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the HSA library has no multi-GPU "
              f"path (asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import chunk_sparse_attention_amd as hsa
    from chunk_sparse_attention_amd import _lib
    import workloads

    wl = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    if args.ceilings:
        print(json.dumps({"ceilings": ceilings(dev)}), flush=True)
        return 0
    if args.only == "decode":
        log("bench: only decode", run_decode(hsa, _lib, workloads, dev, args.generic, args.steps))
        return 0
    if args.only == "decode_step":
        # the decode_1m step alone, --steps times (for counter runs; with --copy-mib the same
        # copy reference as --only step)
        wl3 = workloads.WORKLOADS["decode_1m"]
        x3 = workloads.make_decode_inputs(wl3, seed=0, slab=4)
        q, qs = x3["q"].to(dev), x3["qs"].to(dev)
        Kc, Vc = x3["Kc"].to(dev), x3["Vc"].to(dev)
        del x3
        Kslc3 = hsa.pool(Kc)
        prob3 = hsa.problem(wl3.B, wl3.L, wl3.Hq, wl3.Hkv, wl3.D, wl3.K, wl3.dtype,
                            generic=args.generic)
        ws3 = hsa.workspace(_lib.HSA_OP_DECODE, prob3, dev)
        for _ in range(args.warmup):
            hsa.decode(q, qs, Kc, Vc, Kslc3, wl3.K, generic=args.generic, ws=ws3)
        torch.cuda.synchronize()
        copy_reference(dev, args.copy_mib)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            hsa.decode(q, qs, Kc, Vc, Kslc3, wl3.K, generic=args.generic, ws=ws3)
        e1.record()
        torch.cuda.synchronize()
        log(f"bench: only decode_step: {e0.elapsed_time(e1) / args.steps:.4f} ms per step")
        return 0
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
        # one workspace for both: the backward reuses the forward's tile job lists, key
        # operand and softmax normalisers (HSA_BWD_AFTER_FWD)
        O = hsa.fwd(Q, K, V, idx, w, generic=gen, ws=ws_bwd)
        if ev is not None:
            ev[2].record()
        g = hsa.bwd(Q, K, V, Qs, Kslc, idx, score, w, dO, generic=gen, ws=ws_bwd,
                    after_fwd=True)
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
        run = {"step": step,
               "select": lambda: hsa.select(Qs, K, wl.K, generic=gen),
               "fwd": lambda: hsa.fwd(Q, K, V, idx, w, generic=gen, ws=ws_fwd, out=O),
               "bwd": lambda: hsa.bwd(Q, K, V, Qs, Kslc, idx, score, w, dO, generic=gen,
                                      ws=ws_bwd)}[args.only]
        torch.cuda.synchronize()
        copy_reference(dev, args.copy_mib)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        log(f"bench: only {args.only}: {e0.elapsed_time(e1) / args.steps:.4f} ms per call")
        return 0

    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # the same step captured once in a HIP graph and replayed as many times: how much of the
    # step is launch overhead (reported beside the eager figure, not as it)
    graph_ms = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        del graph
        log(f"bench: graph replay {graph_ms:.4f} ms per step")
    # the same number of steps again, outside the timed region, for the per-entry and
    # per-kernel split (their event records take a little time of their own)
    log("bench: per-kernel pass")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    hsa.timer_enable(True)
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    hsa.timer_enable(False)
    ktimes = hsa.timer_read()
    names = ["hsa_select", "hsa_fwd", "hsa_bwd"]
    entry_ms = {n: round(sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps, 4)
                for j, n in enumerate(names)}
    # per-step spread (this pass records events, which adds a little to every step)
    per_step = sorted(e[0].elapsed_time(e[3]) for e in evs)
    pct = {f"p{p}": round(per_step[min(len(per_step) - 1, int(p / 100 * len(per_step)))], 4)
           for p in (10, 50, 90)}
    log("bench: per-entry ms", entry_ms)
    counts = kernel_counts(wl, n_slots, fused_backward(wl, gen), chunked_forward(wl, gen),
                           mfma_select(wl, gen))
    kern = {}
    for name, (n, total) in ktimes.items():
        if n == 0:
            continue
        r = roofline(name, counts[name], total / n, measured_traffic(wl.name, name))
        r["launches_per_step"] = round(n / args.steps, 3)
        r["ms_per_step"] = round(total / args.steps, 4)
        kern[name] = r
    log("bench: per-kernel ms/step", {k: v["ms_per_step"] for k, v in kern.items()})
    dominant = max(kern, key=lambda k: kern[k]["ms_per_step"])
    roof = {k: v for k, v in kern[dominant].items() if k not in ("launches_per_step",)}

    # the same step with the softmax chunk weights (HSA_FLAG_SOFTMAX_WEIGHTS): select's extra
    # weight pass and the backward's other chain rule
    def step_softmax():
        Kslc, idx, score, w = hsa.select(Qs, K, wl.K, generic=gen, weights="softmax")
        hsa.fwd(Q, K, V, idx, w, generic=gen, ws=ws_bwd)
        hsa.bwd(Q, K, V, Qs, Kslc, idx, score, w, dO, generic=gen, ws=ws_bwd, after_fwd=True,
                weights="softmax")

    for _ in range(2):
        step_softmax()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_softmax()
    torch.cuda.synchronize()
    sm_ms = (time.perf_counter() - t0) * 1e3 / args.steps

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
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
        "entry_ms": entry_ms,
        "step_ms_spread": pct,
        "kernels": kern,
        "softmax_weights": {"ms_per_step": round(sm_ms, 4),
                            "tokens_per_s": round(tokens / (sm_ms / 1e3), 1)},
    }

    if not args.no_secondary:
        out["secondary"] = run_pass(hsa, _lib, workloads, dev, gen, "fwd_64k",
                                    max(3, args.steps // 4))
        # the backward workload: the same pass at B=2, L=16384, d=64, reported for its
        # hsa_bwd time (selection fixed by the pass's own hsa_select)
        out["backward_b2"] = run_pass(hsa, _lib, workloads, dev, gen, "bwd_16k",
                                      max(3, args.steps // 4))

    if not args.no_decode:
        out["decode"] = run_decode(hsa, _lib, workloads, dev, gen, reps=50,
                                   cpu=not args.no_cpu_baseline)

    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        wl2 = workloads.WORKLOADS["fwd_64k"]
        x2 = workloads.make_inputs(wl2, seed=0, with_grad=False)
        out["cpu_baseline"] = cpu_baseline(wl, x, wl2, x2)
        if out.get("decode") and out["decode"].get("cpu_baseline"):
            out["cpu_baseline"]["configs"]["decode_1m_step"] = out["decode"].pop("cpu_baseline")
        del x2
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
