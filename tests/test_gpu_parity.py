"""GPU parity: libhsa.so (through its C ABI) against the CPU oracle on seeded inputs.

Small cases compare every output element; the full-size workloads compare sampled rows and
chunks the oracle computes one by one.  Tolerances: selection indices bit-exact outside
near-tie rows (see hsa_compare), scores and weights 1e-5, outputs and gradients max-abs 2e-2
for bf16 and 1e-4 for fp32.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from hsa_compare import compare_backward, compare_forward, head_mask, max_abs, npy, say, tol_for

pytestmark = pytest.mark.gpu

W = workloads.Workload


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def hsa():
    import chunk_sparse_attention_amd as m
    return m


def gpu_forward(hsa, x, wl, dev, generic=False, weights="stick"):
    Q, K, V, Qs = (x[k].to(dev) for k in ("Q", "K", "V", "Qs"))
    Kslc, idx, score, w = hsa.select(Qs, K, wl.K, generic=generic, weights=weights)
    O = hsa.fwd(Q, K, V, idx, w, generic=generic)
    return dict(Q=Q, K=K, V=V, Qs=Qs, Kslc=Kslc, idx=idx, score=score, w=w, O=O)


SMALL = [
    W("tiny_fp32", 1, 1024, 4, 1, 64, 64, 4, torch.float32, 1.0, 1.0),
    W("bf16_d64_ragged", 2, 64 * 24 + 37, 16, 2, 64, 64, 8, torch.bfloat16),
    W("bf16_d128_ragged", 1, 64 * 20 + 5, 16, 2, 128, 64, 8, torch.bfloat16),
    W("bf16_g1_k3", 1, 64 * 10, 8, 8, 64, 64, 3, torch.bfloat16),
    W("bf16_g16_k16", 1, 64 * 21, 16, 1, 128, 64, 16, torch.bfloat16),
    W("fp32_k1", 2, 64 * 9 + 1, 4, 2, 64, 64, 1, torch.float32, 1.0, 1.0),
    W("bf16_no_chunk", 1, 50, 8, 2, 64, 64, 4, torch.bfloat16),
    W("planted_d128", 1, 64 * 100, 16, 2, 128, 64, 8, torch.bfloat16, planted=True),
    W("bf16_d64_g4_ragged", 1, 64 * 17 + 9, 8, 2, 64, 64, 6, torch.bfloat16),
    W("bf16_d64_g16_k16", 1, 64 * 19 + 3, 16, 1, 64, 64, 16, torch.bfloat16),
    # one and two query heads per group: 16 and 8 selectors per matrix-core job
    W("bf16_g2_d64_ragged", 1, 64 * 13 + 11, 8, 4, 64, 64, 8, torch.bfloat16),
    W("bf16_g2_d128", 1, 64 * 12 + 3, 4, 2, 128, 64, 5, torch.bfloat16),
    W("bf16_g1_d128_b2", 2, 64 * 9 + 7, 2, 2, 128, 64, 4, torch.bfloat16),
    W("bf16_g1_d64_k16", 1, 64 * 22 + 13, 4, 4, 64, 64, 16, torch.bfloat16),
    W("bf16_g2_d128_k16", 1, 64 * 19 + 1, 8, 4, 128, 64, 16, torch.bfloat16),
]


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "default"])
@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_small_end_to_end(hsa, dev, wl, generic):
    say("case", wl, "generic" if generic else "default")
    orc = oracle.get()
    x = workloads.make_inputs(wl, seed=0)
    g = gpu_forward(hsa, x, wl, dev, generic)
    grads = hsa.bwd(g["Q"], g["K"], g["V"], g["Qs"], g["Kslc"], g["idx"], g["score"], g["w"],
                    x["dO"].to(dev), generic=generic)
    torch.cuda.synchronize()
    f, diff, _ = compare_forward(orc, x, wl, g)
    compare_backward(orc, x, wl, g, f, diff, grads)


@pytest.mark.parametrize("wl", [w for w in SMALL if w.dtype == torch.bfloat16],
                         ids=lambda w: w.name)
def test_backward_after_forward(hsa, dev, wl):
    """Forward and backward on one workspace, the backward reusing the forward's state
    (HSA_BWD_AFTER_FWD): parity with the oracle, and agreement with the stand-alone backward."""
    from chunk_sparse_attention_amd import _lib
    say("case after_fwd", wl)
    orc = oracle.get()
    x = workloads.make_inputs(wl, seed=0)
    Q, K, V, Qs = (x[k].to(dev) for k in ("Q", "K", "V", "Qs"))
    dO = x["dO"].to(dev)
    Kslc, idx, score, w = hsa.select(Qs, K, wl.K)
    prob = hsa.problem(wl.B, wl.L, wl.Hq, wl.Hkv, wl.D, wl.K, wl.dtype)
    ws = hsa.workspace(_lib.HSA_OP_BWD, prob, dev)
    O = hsa.fwd(Q, K, V, idx, w, ws=ws)
    grads = hsa.bwd(Q, K, V, Qs, Kslc, idx, score, w, dO, ws=ws, after_fwd=True)
    alone = hsa.bwd(Q, K, V, Qs, Kslc, idx, score, w, dO)
    torch.cuda.synchronize()
    g = dict(Q=Q, K=K, V=V, Qs=Qs, Kslc=Kslc, idx=idx, score=score, w=w, O=O)
    f, diff, _ = compare_forward(orc, x, wl, g)
    compare_backward(orc, x, wl, g, f, diff, grads)
    for k in ("dQ", "dK", "dV", "dQs"):
        assert max_abs(npy(grads[k]), npy(alone[k])) <= 1e-2, k


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "default"])
@pytest.mark.parametrize("wl", SMALL[1:4], ids=lambda w: w.name)
def test_given_selection(hsa, dev, wl, generic):
    """Attention and backward with one random valid selection given to both sides."""
    say("case", wl, "given selection", generic)
    orc = oracle.get()
    x = workloads.make_inputs(wl, seed=3)
    sel = workloads.make_selection(wl.B, wl.L, wl.Hkv, wl.S, wl.K, seed=4)
    Q, K, V, Qs, dO = (x[k].to(dev) for k in ("Q", "K", "V", "Qs", "dO"))
    idx, score, w = (sel[k].to(dev) for k in ("idx", "score", "w"))
    Kslc = hsa.pool(K)
    O = hsa.fwd(Q, K, V, idx, w, generic=generic)
    grads = hsa.bwd(Q, K, V, Qs, Kslc, idx, score, w, dO, generic=generic)
    torch.cuda.synchronize()
    ks = orc.pool(x["K"], wl.S)
    Oo = orc.attend(x["Q"], x["K"], x["V"], sel["idx"], sel["w"], wl.S)
    tol = tol_for(wl.dtype)
    assert max_abs(npy(O), Oo) <= tol
    o = orc.backward(x["Q"], x["K"], x["V"], x["Qs"], ks, sel["idx"], sel["score"], sel["w"],
                     x["dO"], wl.S)
    rep = {k: max_abs(npy(grads[k]), o[k]) for k in ("dQ", "dK", "dV", "dQs", "dKslc")}
    say("given-selection", wl.name, rep)
    for k, v in rep.items():
        assert v <= tol, (k, v)


def test_graph_replay_matches_eager(hsa, dev):
    """The whole step (select, forward, backward after forward on one workspace) captured in a
    HIP graph: every replay, with eager work between replays, equals the eager step bitwise."""
    from chunk_sparse_attention_amd import _lib
    wl = SMALL[1]
    say("case graph replay", wl)
    x = workloads.make_inputs(wl, seed=8)
    Q, K, V, Qs, dO = (x[k].to(dev) for k in ("Q", "K", "V", "Qs", "dO"))
    prob = hsa.problem(wl.B, wl.L, wl.Hq, wl.Hkv, wl.D, wl.K, wl.dtype)
    ws = hsa.workspace(_lib.HSA_OP_BWD, prob, dev)

    def step():
        Kslc, idx, score, w = hsa.select(Qs, K, wl.K)
        O = hsa.fwd(Q, K, V, idx, w, ws=ws)
        g = hsa.bwd(Q, K, V, Qs, Kslc, idx, score, w, dO, ws=ws, after_fwd=True)
        return [idx, score, w, O] + [g[k] for k in ("dQ", "dK", "dV", "dQs", "dKslc")]

    eager = [t.clone() for t in step()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        static = step()
    for _ in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(static, eager):
            assert torch.equal(a, b)
        step()  # eager work between replays
        torch.cuda.synchronize()


def test_graph_replay_decode(hsa, dev):
    """The decode calls (stick-breaking and softmax weights, ragged lengths, a shared
    selection) captured in one HIP graph: every replay equals the eager calls bitwise."""
    from chunk_sparse_attention_amd import _lib
    ctx = 64 * 40 + 5
    wl = W("decode_graph", 3, ctx, 16, 2, 64, 64, 8, torch.bfloat16)
    x = workloads.make_decode_inputs(wl, seed=60)
    q, qs, Kc, Vc = (x[k].to(dev) for k in ("q", "qs", "Kc", "Vc"))
    Kslc = hsa.pool(Kc)
    lens = torch.tensor([ctx, 64 * 7 + 1, 100], dtype=torch.int32, device=dev)
    prob = hsa.problem(wl.B, ctx, wl.Hq, wl.Hkv, wl.D, wl.K, wl.dtype)
    ws = [hsa.workspace(_lib.HSA_OP_DECODE, prob, dev) for _ in range(3)]
    q2, K2, V2 = torch.stack([q, q.flip(0)]), torch.stack([Kc, Kc]), torch.stack([Vc, Vc])

    def calls():
        O, idx, score, w = hsa.decode(q, qs, Kc, Vc, Kslc, wl.K, ws=ws[0])
        Os, _, _, ws_ = hsa.decode(q, qs, Kc, Vc, Kslc, wl.K, ws=ws[1], weights="softmax")
        Or, ir, _, _ = hsa.decode_ragged(q, qs, Kc, Vc, Kslc, lens, wl.K, ws=ws[2])
        Osh = hsa.decode_shared(q2, K2, V2, idx, w)
        return [O, idx, score, w, Os, ws_, Or, ir, Osh]

    eager = [t.clone() for t in calls()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        static = calls()
    for _ in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(static, eager):
            assert torch.equal(a, b)
        calls()  # eager work between replays
        torch.cuda.synchronize()


def test_backward_bitwise_reproducible(hsa, dev):
    wl = SMALL[1]
    x = workloads.make_inputs(wl, seed=5)
    g = gpu_forward(hsa, x, wl, dev)
    dO = x["dO"].to(dev)
    a = hsa.bwd(g["Q"], g["K"], g["V"], g["Qs"], g["Kslc"], g["idx"], g["score"], g["w"], dO)
    b = hsa.bwd(g["Q"], g["K"], g["V"], g["Qs"], g["Kslc"], g["idx"], g["score"], g["w"], dO)
    torch.cuda.synchronize()
    for k in ("dQ", "dK", "dV", "dQs", "dKslc"):
        assert torch.equal(a[k], b[k]), k


def test_fold_flag(hsa, dev):
    """Without HSA_BWD_FOLD_KSLC, dK lacks exactly dKslc/S on every row of each chunk."""
    wl = SMALL[5]
    x = workloads.make_inputs(wl, seed=6)
    g = gpu_forward(hsa, x, wl, dev)
    dO = x["dO"].to(dev)
    a = hsa.bwd(g["Q"], g["K"], g["V"], g["Qs"], g["Kslc"], g["idx"], g["score"], g["w"], dO)
    b = hsa.bwd(g["Q"], g["K"], g["V"], g["Qs"], g["Kslc"], g["idx"], g["score"], g["w"], dO,
                fold=False)
    torch.cuda.synchronize()
    nC = wl.nC
    fold = a["dKslc"].repeat_interleave(64, dim=1) / 64
    d = (a["dK"][:, :nC * 64] - b["dK"][:, :nC * 64]).double()
    assert (d - fold.double()).abs().max().item() <= 1e-5
    assert torch.equal(a["dV"], b["dV"]) and torch.equal(a["dQ"], b["dQ"])


@pytest.mark.parametrize("case", ["qs_zero", "qs_half_zero", "equal_chunks", "qs_large",
                                  "qs_nan", "qs_inf", "k_nan", "signed_zero", "negative_scale",
                                  "tiny_scale"])
@pytest.mark.parametrize("d", [64, 128])
def test_select_degenerate(hsa, dev, case, d):
    """Exact ties, extreme magnitudes and values that are not ordinary numbers: the ranking
    must still equal the oracle's bit for bit (ties go to the lower chunk index, a NaN score
    ranks as -inf, -0 as +0), whatever path the kernel takes."""
    wl = W("sel_" + case, 1, 64 * 70 + 7, 8, 2, d, 64, 8, torch.bfloat16)
    say("case select", case, d)
    x = workloads.make_inputs(wl, seed=5, with_grad=False)
    Qs, K = x["Qs"].clone(), x["K"].clone()
    nan, inf = float("nan"), float("inf")
    if case == "qs_zero":
        Qs.zero_()
    elif case == "qs_half_zero":
        Qs[:, ::2] = 0
    elif case == "equal_chunks":
        nC = wl.L // 64
        K[:, :nC * 64] = K[:, :64].repeat(1, nC, 1, 1)
    elif case == "qs_large":
        Qs = (Qs.float() * 2.0 ** 100).to(torch.bfloat16)
    elif case == "qs_nan":  # whole rows and single components
        Qs[0, 300:4000:37, 0, :] = nan
        Qs[0, 150:4400:23, 1, 5] = nan
    elif case == "qs_inf":  # scores +-inf, or NaN where a key component is 0
        Qs[0, 200:4400:29, 0, 3] = inf
        Qs[0, 180:4400:31, 1, 7] = -inf
        K[0, 64 * 11:64 * 12, 0, 3] = 0  # chunk 11's key is 0 there: inf * 0
    elif case == "k_nan":  # chunk keys with NaN or inf components
        K[0, 64 * 5 + 7, 0, 10] = nan
        K[0, 64 * 9 + 1, 1, 3] = inf
        K[0, 64 * 30 + 2, 0, 1] = -inf
    elif case == "signed_zero":  # rows whose every score rounds to +0 or -0 in fp32
        Qs[0, 500:4000:13, :, :] = 0
        Qs[0, 500:4000:13, :, 0] = 2.0 ** -133
    # a negative selection scale reverses the ranking (the filter's bound takes |scale|);
    # a tiny one makes every score subnormal in fp32, where rounding ties many chunks
    sel = {"signed_zero": 2.0 ** -20, "negative_scale": -0.125, "tiny_scale": 2.0 ** -140}.get(case)
    Kslc, idx, score, w = hsa.select(Qs.to(dev), K.to(dev), wl.K, sel_scale=sel)
    torch.cuda.synchronize()
    orc = oracle.get()
    ks = orc.pool(K, 64)
    assert np.array_equal(npy(Kslc), ks, equal_nan=True)
    oi, osc, ow = orc.select(Qs, ks, 64, wl.K, sel_scale=sel)
    if case == "signed_zero":  # the planted rows rank their chunks in index order
        t = np.arange(500, 4000, 13)
        valid = oi[0, t] >= 0
        assert np.all(osc[0, t][valid] == 0) and np.any(np.signbit(osc[0, t][valid]))
        assert np.array_equal(oi[0, t, :, 0], np.zeros_like(oi[0, t, :, 0]))
    assert np.array_equal(npy(idx), oi)
    sc = npy(score)
    fin = np.isfinite(osc)
    assert np.array_equal(np.isfinite(sc), fin)
    assert not np.isnan(sc).any() and not np.isnan(npy(w)).any()
    assert np.array_equal(sc[~fin], osc[~fin])  # the same infinities
    assert np.array_equal(sc[fin].astype(np.float32), osc[fin].astype(np.float32))
    assert max_abs(npy(w), ow) <= 1e-5


@pytest.mark.parametrize("ctx", [40, 64, 64 * 7 + 13, 64 * 33])
@pytest.mark.parametrize("generic", [True, False], ids=["generic", "default"])
def test_decode_small(hsa, dev, ctx, generic):
    wl = W("decode_small", 3, ctx, 16, 2, 64, 64, 8, torch.bfloat16)
    say("case decode", ctx, generic)
    x = workloads.make_decode_inputs(wl, seed=7, ctx=ctx)
    q, qs, Kc, Vc = (x[k].to(dev) for k in ("q", "qs", "Kc", "Vc"))
    Kslc = hsa.pool(Kc)
    O, idx, score, w = hsa.decode(q, qs, Kc, Vc, Kslc, wl.K, generic=generic)
    torch.cuda.synchronize()
    orc = oracle.get()
    ks = orc.pool(x["Kc"], 64)
    assert np.array_equal(npy(Kslc), ks)
    d = orc.decode(x["q"], x["qs"], x["Kc"], x["Vc"], ks, 64, wl.K)
    assert np.array_equal(npy(idx), d["idx"])
    assert max_abs(npy(w), d["w"]) <= 1e-5
    assert max_abs(npy(O), d["O"]) <= 2e-2


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "default"])
def test_decode_nonfinite_scores(hsa, dev, generic):
    """Decode with selection queries that are not ordinary numbers: a NaN score ranks as -inf
    (the slots take chunks in index order with weight 0, so the heads' output is 0) and an
    +inf score takes all of the stick."""
    ctx = 64 * 33 + 5
    wl = W("decode_nonfinite", 3, ctx, 16, 2, 64, 64, 8, torch.bfloat16)
    say("case decode nonfinite", generic)
    x = workloads.make_decode_inputs(wl, seed=9, ctx=ctx)
    qs = x["qs"].clone()
    qs[1, 0, :] = float("nan")
    qs[2, 1, 4] = float("inf")
    q, Kc, Vc = (x[k].to(dev) for k in ("q", "Kc", "Vc"))
    Kslc = hsa.pool(Kc)
    O, idx, score, w = hsa.decode(q, qs.to(dev), Kc, Vc, Kslc, wl.K, generic=generic)
    torch.cuda.synchronize()
    orc = oracle.get()
    ks = orc.pool(x["Kc"], 64)
    d = orc.decode(x["q"], qs, x["Kc"], x["Vc"], ks, 64, wl.K)
    assert list(d["idx"][1, 0]) == list(range(8)) and np.all(d["w"][1, 0] == 0)
    assert np.isposinf(d["score"][2, 1, 0]) and d["w"][2, 1, 0] == 1.0
    assert np.array_equal(npy(idx), d["idx"])
    sc = npy(score)
    assert not np.isnan(sc).any()
    assert np.array_equal(sc[~np.isfinite(d["score"])], d["score"][~np.isfinite(d["score"])])
    assert max_abs(npy(w), d["w"]) <= 1e-5
    assert max_abs(npy(O), d["O"]) <= 2e-2
    assert np.all(npy(O)[1, :8] == 0)


@pytest.mark.parametrize("k", [8, 16])
@pytest.mark.parametrize("case", ["nan_query", "equal_chunks"])
def test_decode_ties(hsa, dev, case, k):
    """Decode where many chunks tie (a NaN selection query ranks every chunk as -inf; equal
    chunk keys give every chunk the same score): more tied keys than one wave holds reach
    both the scan blocks' and the merge's ranking, which must still give the oracle's
    ranks (ties to the lower chunk index) bit for bit."""
    ctx = 64 * 5200 + 7  # six scan blocks of 1024 chunks
    wl = W("decode_ties", 2, ctx, 16, 2, 64, 64, k, torch.bfloat16)
    say("case decode ties", case, k)
    x = workloads.make_decode_inputs(wl, seed=13, ctx=ctx)
    qs, Kc = x["qs"].clone(), x["Kc"].clone()
    if case == "nan_query":
        qs[0, 1, :] = float("nan")
        qs[1, 0, 3] = float("nan")
    else:
        nC = ctx // 64
        Kc[1, :nC * 64] = Kc[1, :64].repeat(nC, 1, 1)
    q, Vc = x["q"].to(dev), x["Vc"].to(dev)
    Kd = Kc.to(dev)
    Kslc = hsa.pool(Kd)
    O, idx, score, w = hsa.decode(q, qs.to(dev), Kd, Vc, Kslc, wl.K)
    torch.cuda.synchronize()
    orc = oracle.get()
    ks = orc.pool(Kc, 64)
    d = orc.decode(x["q"], qs, Kc, x["Vc"], ks, 64, wl.K)
    if case == "nan_query":
        assert list(d["idx"][0, 1]) == list(range(k))
    else:
        assert np.array_equal(d["idx"][1], np.tile(np.arange(k), (2, 1)))
    assert np.array_equal(npy(idx), d["idx"])
    sc = npy(score)
    fin = np.isfinite(d["score"])
    assert np.array_equal(sc[~fin], d["score"][~fin])
    assert np.array_equal(sc[fin].astype(np.float32), d["score"][fin].astype(np.float32))
    assert max_abs(npy(w), d["w"]) <= 1e-5
    assert max_abs(npy(O), d["O"]) <= 2e-2


SOFTMAX_CASES = [w for w in SMALL if w.name in ("tiny_fp32", "bf16_d64_ragged", "bf16_d128_ragged",
                                               "bf16_g1_k3", "fp32_k1", "bf16_d64_g16_k16",
                                               "bf16_g2_d128")]


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "default"])
@pytest.mark.parametrize("wl", SOFTMAX_CASES, ids=lambda w: w.name)
def test_softmax_weights_end_to_end(hsa, dev, wl, generic):
    """HSA_FLAG_SOFTMAX_WEIGHTS: selection, softmax chunk weights, attention and the
    backward through the softmax chain rule against the oracle's softmax mode."""
    say("case softmax weights", wl, "generic" if generic else "default")
    orc = oracle.get()
    x = workloads.make_inputs(wl, seed=3)
    g = gpu_forward(hsa, x, wl, dev, generic, weights="softmax")
    grads = hsa.bwd(g["Q"], g["K"], g["V"], g["Qs"], g["Kslc"], g["idx"], g["score"], g["w"],
                    x["dO"].to(dev), generic=generic, weights="softmax")
    torch.cuda.synchronize()
    f, diff, _ = compare_forward(orc, x, wl, g, weights="softmax")
    w = npy(g["w"])
    rows = (npy(g["idx"]) >= 0).any(-1)
    assert np.allclose(w.sum(-1)[rows], 1.0, atol=1e-5)
    compare_backward(orc, x, wl, g, f, diff, grads, weights="softmax")


@pytest.mark.parametrize("ctx", [40, 64 * 7 + 13, 64 * 33])
@pytest.mark.parametrize("generic", [True, False], ids=["generic", "default"])
def test_decode_softmax_weights(hsa, dev, ctx, generic):
    wl = W("decode_softmax", 3, ctx, 16, 2, 64, 64, 8, torch.bfloat16)
    say("case decode softmax", ctx, generic)
    x = workloads.make_decode_inputs(wl, seed=8, ctx=ctx)
    q, qs, Kc, Vc = (x[k].to(dev) for k in ("q", "qs", "Kc", "Vc"))
    Kslc = hsa.pool(Kc)
    O, idx, score, w = hsa.decode(q, qs, Kc, Vc, Kslc, wl.K, generic=generic, weights="softmax")
    torch.cuda.synchronize()
    orc = oracle.get()
    ks = orc.pool(x["Kc"], 64)
    d = orc.decode(x["q"], x["qs"], x["Kc"], x["Vc"], ks, 64, wl.K, weights="softmax")
    assert np.array_equal(npy(idx), d["idx"])
    assert max_abs(npy(w), d["w"]) <= 1e-5
    assert max_abs(npy(O), d["O"]) <= 2e-2


LAYER_CASES = [w for w in SMALL if w.name in ("tiny_fp32", "bf16_d64_ragged", "bf16_d128_ragged",
                                             "bf16_g2_d64_ragged")]


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "default"])
@pytest.mark.parametrize("wl", LAYER_CASES, ids=lambda w: w.name)
def test_fwd_layers(hsa, dev, wl, generic):
    """Three layers sharing one selection: each layer's output equals hsa_fwd's on that layer
    bit for bit (the index is built once) and the oracle's."""
    say("case fwd layers", wl, generic)
    n = 3
    xs = [workloads.make_inputs(wl, seed=20 + l, with_grad=False) for l in range(n)]
    Q = torch.stack([x["Q"] for x in xs]).to(dev)
    K = torch.stack([x["K"] for x in xs]).to(dev)
    V = torch.stack([x["V"] for x in xs]).to(dev)
    _, idx, _, w = hsa.select(xs[0]["Qs"].to(dev), K[0], wl.K, generic=generic)
    O = hsa.fwd_layers(Q, K, V, idx, w, generic=generic)
    torch.cuda.synchronize()
    orc = oracle.get()
    for l in range(n):
        ref = hsa.fwd(Q[l], K[l], V[l], idx, w, generic=generic)
        torch.cuda.synchronize()
        assert torch.equal(O[l], ref), l
        o = orc.attend(xs[l]["Q"], xs[l]["K"], xs[l]["V"], npy(idx), npy(w), wl.S)
        assert max_abs(npy(O[l]), o) <= tol_for(wl.dtype), l


@pytest.mark.parametrize("wl", [w for w in LAYER_CASES if w.dtype == torch.bfloat16],
                         ids=lambda w: w.name)
def test_fwd_layers_then_backward(hsa, dev, wl):
    """After hsa_fwd_layers the workspace holds the last layer's forward state: a backward of
    that layer with HSA_BWD_AFTER_FWD equals, bit for bit, the one after hsa_fwd of that
    layer alone."""
    from chunk_sparse_attention_amd import _lib
    say("case fwd_layers then backward", wl)
    n = 3
    xs = [workloads.make_inputs(wl, seed=70 + l) for l in range(n)]
    Q = torch.stack([x["Q"] for x in xs]).to(dev)
    K = torch.stack([x["K"] for x in xs]).to(dev)
    V = torch.stack([x["V"] for x in xs]).to(dev)
    Qs, dO = xs[0]["Qs"].to(dev), xs[-1]["dO"].to(dev)
    Kslc, idx, score, w = hsa.select(Qs, K[0], wl.K)
    prob = hsa.problem(wl.B, wl.L, wl.Hq, wl.Hkv, wl.D, wl.K, wl.dtype)
    ws = hsa.workspace(_lib.HSA_OP_BWD, prob, dev)
    hsa.fwd_layers(Q, K, V, idx, w, ws=ws)
    got = hsa.bwd(Q[-1], K[-1], V[-1], Qs, Kslc, idx, score, w, dO, ws=ws, after_fwd=True)
    ws2 = hsa.workspace(_lib.HSA_OP_BWD, prob, dev)
    hsa.fwd(Q[-1], K[-1], V[-1], idx, w, ws=ws2)
    ref = hsa.bwd(Q[-1], K[-1], V[-1], Qs, Kslc, idx, score, w, dO, ws=ws2, after_fwd=True)
    torch.cuda.synchronize()
    for k in ("dQ", "dK", "dV", "dQs"):
        assert torch.equal(got[k], ref[k]), k


def test_fwd_layers_token_tiles(hsa, dev):
    """Past 16384 chunks the forward runs on token tiles; their job lists are built once for
    the stack: each layer equals hsa_fwd's (whose parity the token-tile test checks)."""
    wl = W("bf16_16400_chunks", 1, 64 * 16400 + 17, 8, 2, 64, 64, 4, torch.bfloat16)
    say("case fwd layers token tiles", wl)
    xs = [workloads.make_inputs(wl, seed=30 + l, with_grad=False) for l in range(2)]
    Q = torch.stack([x["Q"] for x in xs]).to(dev)
    K = torch.stack([x["K"] for x in xs]).to(dev)
    V = torch.stack([x["V"] for x in xs]).to(dev)
    _, idx, _, w = hsa.select(xs[0]["Qs"].to(dev), K[0], wl.K)
    O = hsa.fwd_layers(Q, K, V, idx, w)
    for l in range(2):
        ref = hsa.fwd(Q[l], K[l], V[l], idx, w)
        torch.cuda.synchronize()
        assert torch.equal(O[l], ref), l


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_decode_shared(hsa, dev, dtype):
    """Layers reusing layer 0's decode selection: layer 0 reproduces its own decode bit for
    bit, and every layer equals the oracle's attention of its query over the given chunks."""
    ctx, n = 64 * 21 + 9, 3
    wl = W("decode_shared", 2, ctx, 16, 2, 64, 64, 8, dtype)
    say("case decode shared", dtype)
    xs = [workloads.make_decode_inputs(wl, seed=40 + l) for l in range(n)]
    q = torch.stack([x["q"] for x in xs]).to(dev)
    Kc = torch.stack([x["Kc"] for x in xs]).to(dev)
    Vc = torch.stack([x["Vc"] for x in xs]).to(dev)
    qs = xs[0]["qs"].to(dev)
    O0, idx, _, w = hsa.decode(q[0], qs, Kc[0], Vc[0], hsa.pool(Kc[0]), wl.K)
    O = hsa.decode_shared(q, Kc, Vc, idx, w)
    torch.cuda.synchronize()
    assert torch.equal(O[0], O0)
    orc = oracle.get()
    B, Hkv, K = idx.shape
    # the decode row as row ctx of a sequence of ctx + 1 tokens, the only row computed
    for l in range(n):
        Qf = torch.zeros((B, ctx + 1, wl.Hq, wl.D), dtype=dtype)
        Qf[:, ctx] = xs[l]["q"]
        pad = torch.zeros((B, 1, Hkv, wl.D), dtype=dtype)
        Kf = torch.cat([xs[l]["Kc"], pad], 1)
        Vf = torch.cat([xs[l]["Vc"], pad], 1)
        idf = np.full((B, ctx + 1, Hkv, K), -1, np.int32)
        wf = np.zeros((B, ctx + 1, Hkv, K))
        idf[:, ctx] = npy(idx)
        wf[:, ctx] = npy(w)
        mask = np.zeros((B, ctx + 1), np.uint8)
        mask[:, ctx] = 1
        o = orc.attend(Qf, Kf, Vf, idf, wf, 64, row_mask=mask)
        assert max_abs(npy(O[l]), o[:, ctx]) <= tol_for(dtype), l


def test_decode_shared_masked_slots(hsa, dev):
    """A given selection with a masked slot between valid ones and an index past the cache:
    both slots add nothing, the others are summed in slot order."""
    ctx = 64 * 9 + 5
    wl = W("decode_shared_masks", 2, ctx, 8, 2, 64, 64, 4, torch.bfloat16)
    x = workloads.make_decode_inputs(wl, seed=50)
    q, Kc, Vc = (x[k].to(dev) for k in ("q", "Kc", "Vc"))
    idx = torch.tensor([[[3, -1, 7, 2], [0, 8, 99, 5]], [[1, 2, -1, -1], [6, 4, 3, 0]]],
                       dtype=torch.int32)
    w = torch.tensor([[[0.4, 0.3, 0.2, 0.1], [0.25, 0.25, 0.3, 0.2]],
                      [[0.5, 0.5, 0.0, 0.0], [0.1, 0.2, 0.3, 0.4]]], dtype=torch.float32)
    O = hsa.decode_shared(q[None], Kc[None], Vc[None], idx.to(dev), w.to(dev))
    torch.cuda.synchronize()
    eff = torch.where(idx < ctx // 64, idx, torch.full_like(idx, -1))  # 99 is past the cache
    B, Hkv, K = idx.shape
    Qf = torch.zeros((B, ctx + 1, wl.Hq, wl.D), dtype=wl.dtype)
    Qf[:, ctx] = x["q"]
    pad = torch.zeros((B, 1, Hkv, wl.D), dtype=wl.dtype)
    idf = np.full((B, ctx + 1, Hkv, K), -1, np.int32)
    wf = np.zeros((B, ctx + 1, Hkv, K))
    idf[:, ctx] = eff.numpy()
    wf[:, ctx] = np.where(eff.numpy() >= 0, w.numpy(), 0.0)
    mask = np.zeros((B, ctx + 1), np.uint8)
    mask[:, ctx] = 1
    o = oracle.get().attend(Qf, torch.cat([x["Kc"], pad], 1), torch.cat([x["Vc"], pad], 1), idf,
                            wf, 64, row_mask=mask)
    assert max_abs(npy(O[0]), o[:, ctx]) <= 2e-2


@pytest.mark.parametrize("K", [8, 12], ids=["k8", "k12"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_decode_shared_host_kv(hsa, dev, dtype, K):
    """Shared-selection decode over pinned host caches: each head's sums are taken as with
    device caches (only the grouping of heads into blocks differs), so the results are equal
    bit for bit; pageable memory is refused."""
    ctx, n = 64 * 30 + 17, 3
    wl = W("decode_shared_host", 2, ctx, 16, 2, 64, 64, K, dtype)
    say("case decode shared host kv", dtype, K)
    xs = [workloads.make_decode_inputs(wl, seed=60 + l) for l in range(n)]
    q = torch.stack([x["q"] for x in xs]).to(dev)
    Kh = torch.stack([x["Kc"] for x in xs]).pin_memory()
    Vh = torch.stack([x["Vc"] for x in xs]).pin_memory()
    Kc, Vc = Kh.to(dev), Vh.to(dev)
    _, idx, _, w = hsa.decode(q[0], xs[0]["qs"].to(dev), Kc[0], Vc[0], hsa.pool(Kc[0]), K)
    ref = hsa.decode_shared(q, Kc, Vc, idx, w)
    got = hsa.decode_shared(q, Kh, Vh, idx, w)
    # views that start inside the pinned allocations
    tail = hsa.decode_shared(q[1:], Kh[1:], Vh[1:], idx, w)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(tail, ref[1:])
    from chunk_sparse_attention_amd import _lib
    prob = hsa.problem(2, ctx, 16, 2, 64, K, dtype)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    Kp = Kh.clone()  # pageable host memory
    for kc in (Kp, Kc):  # pageable host memory, then device memory
        st = _lib.lib().hsa_decode_shared_host_kv(
            ctypes.byref(prob), n, P(q), P(kc), P(kc), P(idx), P(w), P(got),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == _lib.HSA_ERR_INVALID_ARG, _lib.lib().hsa_last_error()
    with pytest.raises(ValueError):
        hsa.decode_shared(q, Kp, Vh.clone(), idx, w)


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "default"])
def test_decode_ragged(hsa, dev, generic):
    """Sequences of different lengths in one cache: each sequence's result equals hsa_decode
    on its own prefix bit for bit, and the oracle's; a sequence of length 0 (or a negative
    length, which counts as 0) selects nothing: every slot masked, O zero."""
    cap = 64 * 40 + 5
    lens = [0, 40, 64 * 7 + 13, -7, 64 * 33, cap]
    wl = W("decode_ragged", len(lens), cap, 16, 2, 64, 64, 8, torch.bfloat16)
    say("case decode ragged", lens, generic)
    x = workloads.make_decode_inputs(wl, seed=12)
    q, qs, Kc, Vc = (x[k].to(dev) for k in ("q", "qs", "Kc", "Vc"))
    Kslc = hsa.pool(Kc)
    ctx_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    got = hsa.decode_ragged(q, qs, Kc, Vc, Kslc, ctx_lens, wl.K, generic=generic)
    torch.cuda.synchronize()
    orc = oracle.get()
    for b, n in enumerate(lens):
        if n <= 0:
            assert torch.all(got[1][b] == -1) and torch.all(got[3][b] == 0)
            assert torch.all(torch.isneginf(got[2][b])) and torch.all(got[0][b] == 0)
            continue
        Kb, Vb = Kc[b:b + 1, :n].contiguous(), Vc[b:b + 1, :n].contiguous()
        ref = hsa.decode(q[b:b + 1], qs[b:b + 1], Kb, Vb, hsa.pool(Kb), wl.K, generic=generic)
        torch.cuda.synchronize()
        for a, r in zip(got, ref):
            assert torch.equal(a[b:b + 1], r), (b, n)
        xb = {k: x[k][b:b + 1] for k in ("q", "qs")}
        kb, vb = x["Kc"][b:b + 1, :n], x["Vc"][b:b + 1, :n]
        d = orc.decode(xb["q"], xb["qs"], kb, vb, orc.pool(kb, 64), 64, wl.K)
        assert np.array_equal(npy(got[1][b:b + 1]), d["idx"]), (b, n)
        assert max_abs(npy(got[3][b:b + 1]), d["w"]) <= 1e-5
        assert max_abs(npy(got[0][b:b + 1]), d["O"]) <= 2e-2


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_pool_chunks(hsa, dev, dtype):
    """Pooling listed chunks only reproduces the full pooling of those chunks bit for bit and
    leaves the others alone."""
    gen = torch.Generator().manual_seed(4)
    B, L, Hkv, D = 3, 64 * 20 + 7, 2, 64
    K = (torch.randn((B, L, Hkv, D), generator=gen) * 0.5).to(dtype).to(dev)
    full = hsa.pool(K)
    ids = torch.tensor([[3, -1, 19], [0, 7, 25], [-1, -1, 12]], dtype=torch.int32)
    Kslc = full.clone()
    for b in range(B):
        for c in ids[b].tolist():
            if 0 <= c < L // 64:
                Kslc[b, c] = 0
    hsa.pool_chunks(K, Kslc, ids.to(dev))
    torch.cuda.synchronize()
    assert torch.equal(Kslc, full)


def test_decode_incremental(hsa, dev):
    """A decoder loop: sequences grow one token per step; when one completes a chunk, that
    chunk's key is pooled into the resident table (hsa_pool_chunks) and the next step may
    select it.  Every step equals the oracle's decode on each sequence's prefix."""
    cap = 64 * 12
    lens = [64 * 5 + 62, 64 * 3 + 63]
    wl = W("decode_incremental", len(lens), cap, 8, 2, 64, 64, 4, torch.bfloat16)
    x = workloads.make_decode_inputs(wl, seed=13)
    q, qs, Kc, Vc = (x[k].to(dev) for k in ("q", "qs", "Kc", "Vc"))
    Kslc = hsa.pool(Kc)
    for b, n in enumerate(lens):  # only the chunks complete at the start are in the table
        Kslc[b, n // 64:] = 0
    orc = oracle.get()
    for step in range(4):
        ctx_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
        O, idx, _, w = hsa.decode_ragged(q, qs, Kc, Vc, Kslc, ctx_lens, wl.K)
        torch.cuda.synchronize()
        for b, n in enumerate(lens):
            kb, vb = x["Kc"][b:b + 1, :n], x["Vc"][b:b + 1, :n]
            d = orc.decode(x["q"][b:b + 1], x["qs"][b:b + 1], kb, vb, orc.pool(kb, 64), 64, wl.K)
            assert np.array_equal(npy(idx[b:b + 1]), d["idx"]), (step, b, n)
            assert max_abs(npy(w[b:b + 1]), d["w"]) <= 1e-5
            assert max_abs(npy(O[b:b + 1]), d["O"]) <= 2e-2
        # one more token per sequence; a completed chunk joins the table
        lens = [n + 1 for n in lens]
        done = [[n // 64 - 1 if n % 64 == 0 else -1] for n in lens]
        hsa.pool_chunks(Kc, Kslc, torch.tensor(done, dtype=torch.int32, device=dev))


@pytest.mark.parametrize("ctx", [64 * 7 + 13, 64 * 33])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_decode_host_kv(hsa, dev, ctx, dtype):
    """The caches in pinned host memory: the same kernels read the selected chunks across the
    host link, so the results equal those with device caches bit for bit, and the oracle's."""
    wl = W("decode_host_kv", 3, ctx, 16, 2, 64, 64, 8, dtype)
    say("case decode host kv", ctx, dtype)
    x = workloads.make_decode_inputs(wl, seed=9, ctx=ctx)
    q, qs, Kc, Vc = (x[k].to(dev) for k in ("q", "qs", "Kc", "Vc"))
    Kh, Vh = x["Kc"].pin_memory(), x["Vc"].pin_memory()
    Kslc = hsa.pool(Kc)
    ref = hsa.decode(q, qs, Kc, Vc, Kslc, wl.K)
    got = hsa.decode_host_kv(q, qs, Kh, Vh, Kslc, wl.K)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    orc = oracle.get()
    ks = orc.pool(x["Kc"], 64)
    d = orc.decode(x["q"], x["qs"], x["Kc"], x["Vc"], ks, 64, wl.K)
    assert np.array_equal(npy(got[1]), d["idx"])
    assert max_abs(npy(got[3]), d["w"]) <= 1e-5
    assert max_abs(npy(got[0]), d["O"]) <= tol_for(dtype)


def test_decode_host_kv_rejects_other_memory(hsa, dev):
    """Pageable host memory and device memory are refused before anything is enqueued."""
    from chunk_sparse_attention_amd import _lib
    wl = W("decode_host_kv", 1, 256, 8, 2, 64, 64, 2, torch.bfloat16)
    x = workloads.make_decode_inputs(wl, seed=1)
    q, qs, Kc = (x[k].to(dev) for k in ("q", "qs", "Kc"))
    Kslc = hsa.pool(Kc)
    prob = hsa.problem(1, 256, 8, 2, 64, 2, torch.bfloat16)
    out = torch.empty((1, 8, 64), dtype=torch.bfloat16, device=dev)
    small = torch.empty((1, 2, 2), dtype=torch.float32, device=dev)
    idx = torch.empty((1, 2, 2), dtype=torch.int32, device=dev)
    ws = hsa.workspace(_lib.HSA_OP_DECODE, prob, dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    L = _lib.lib()
    for kc in (x["Kc"], Kc):  # pageable host memory, then device memory
        st = L.hsa_decode_host_kv(ctypes.byref(prob), P(q), P(qs), P(kc), P(kc), P(Kslc),
                                  P(out), P(idx), None, P(small), P(ws), ws.numel(),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == _lib.HSA_ERR_INVALID_ARG, L.hsa_last_error()
        assert b"Kcache" in L.hsa_last_error()
    # the library still works afterwards
    O, i2, _, _ = hsa.decode(q, qs, Kc, x["Vc"].to(dev), Kslc, 2)
    torch.cuda.synchronize()
    assert O.shape == (1, 8, 64)


@pytest.mark.parametrize("shape", [
    ("f32_d64_g4_k4", torch.float32, 64, 4, 1, 4, 1024 + 17),
    ("bf16_d128_g16_k16", torch.bfloat16, 128, 32, 2, 16, 64 * 40 + 5),
    ("bf16_d64_g1_k1", torch.bfloat16, 64, 8, 8, 1, 64 * 20),
    ("bf16_d64_g2_k8", torch.bfloat16, 64, 4, 2, 8, 64 * 33 + 9),
    ("f32_d128_g4_k3", torch.float32, 128, 16, 4, 3, 64 * 9),
    ("f32_d128_g4_k12", torch.float32, 128, 8, 2, 12, 64 * 30 + 3),
], ids=lambda s: s[0])
@pytest.mark.parametrize("generic", [True, False], ids=["generic", "default"])
def test_decode_shapes(hsa, dev, shape, generic):
    name, dt, D, Hq, Hkv, K, ctx = shape
    wl = W("decode_" + name, 2, ctx, Hq, Hkv, D, 64, K, dt)
    say("case decode", name, ctx, generic)
    x = workloads.make_decode_inputs(wl, seed=11, ctx=ctx)
    q, qs, Kc, Vc = (x[k].to(dev) for k in ("q", "qs", "Kc", "Vc"))
    Kslc = hsa.pool(Kc)
    O, idx, score, w = hsa.decode(q, qs, Kc, Vc, Kslc, K, generic=generic)
    torch.cuda.synchronize()
    orc = oracle.get()
    ks = orc.pool(x["Kc"], 64)
    d = orc.decode(x["q"], x["qs"], x["Kc"], x["Vc"], ks, 64, K)
    assert np.array_equal(npy(idx), d["idx"])
    sc = npy(score)
    fin = np.isfinite(d["score"])
    assert np.array_equal(np.isfinite(sc), fin)
    assert max_abs(sc, d["score"], mask=fin) <= 1e-5
    assert max_abs(npy(w), d["w"]) <= 1e-5
    assert max_abs(npy(O), d["O"]) <= tol_for(dt)


# ---- full-size workloads, sampled --------------------------------------------------------

def _sample_rows(wl, n, seed):
    rng = np.random.default_rng(seed)
    m = np.zeros((wl.B, wl.L), np.uint8)
    for b in range(wl.B):
        ts = rng.choice(wl.L, size=min(n, wl.L), replace=False)
        m[b, ts] = 1
        m[b, [0, wl.S - 1, wl.S, 2 * wl.S - 1, wl.L - 1]] = 1  # boundaries
    return m


@pytest.mark.parametrize("name", ["fwd_16k", "fwd_64k"])
def test_full_forward_sampled(hsa, dev, name):
    wl = workloads.WORKLOADS[name]
    say("case full forward", name)
    x = workloads.make_inputs(wl, seed=0, with_grad=False)
    g = gpu_forward(hsa, x, wl, dev)
    torch.cuda.synchronize()
    mask = _sample_rows(wl, 384, seed=1)
    compare_forward(oracle.get(), x, wl, g, row_mask=mask)


@pytest.mark.parametrize("D,Hq,Hkv", [(64, 16, 4), (128, 16, 1)], ids=["d64", "d128"])
def test_select_k16_many_chunks(hsa, dev, D, Hq, Hkv):
    """K = 16 over up to 260 earlier chunks: the selection filter keeps only K/4 + 2 scores
    per lane for its threshold, so its bound is loosest here; selection is compared on every
    row, outputs on sampled rows."""
    wl = W(f"bf16_k16_d{D}", 1, 64 * 260 + 11, Hq, Hkv, D, 64, 16, torch.bfloat16)
    say("case select K=16", wl)
    x = workloads.make_inputs(wl, seed=21, with_grad=False)
    g = gpu_forward(hsa, x, wl, dev)
    torch.cuda.synchronize()
    compare_forward(oracle.get(), x, wl, g, out_mask=_sample_rows(wl, 256, seed=22))


def test_long_sequence_token_tile_forward(hsa, dev):
    """Past 16384 chunks the forward uses its token-tile kernels (job lists per token tile,
    rounds of jobs, LDS accumulation): parity on sampled rows of a sequence of 16400 chunks."""
    wl = W("bf16_16400_chunks", 1, 64 * 16400 + 17, 8, 2, 64, 64, 4, torch.bfloat16)
    say("case token-tile forward", wl)
    x = workloads.make_inputs(wl, seed=6, with_grad=False)
    g = gpu_forward(hsa, x, wl, dev)
    torch.cuda.synchronize()
    mask = _sample_rows(wl, 96, seed=7)
    compare_forward(oracle.get(), x, wl, g, row_mask=mask)


def test_full_backward_sampled(hsa, dev):
    wl = workloads.WORKLOADS["bwd_16k"]
    say("case full backward bwd_16k")
    x = workloads.make_inputs(wl, seed=0)
    g = gpu_forward(hsa, x, wl, dev)
    grads = hsa.bwd(g["Q"], g["K"], g["V"], g["Qs"], g["Kslc"], g["idx"], g["score"], g["w"],
                    x["dO"].to(dev))
    torch.cuda.synchronize()
    orc = oracle.get()
    f, diff, _ = compare_forward(orc, x, wl, g)  # the selection on every row
    tm = _sample_rows(wl, 48, seed=2)
    rng = np.random.default_rng(3)
    cm = np.zeros((wl.B, wl.nC), np.uint8)
    for b in range(wl.B):
        cm[b, rng.choice(wl.nC, size=6, replace=False)] = 1
        cm[b, [0, 1, wl.nC - 2, wl.nC - 1]] = 1
    compare_backward(orc, x, wl, g, f, diff, grads, tok_mask=tm, chunk_mask=cm)


@pytest.mark.parametrize("name", ["fwd_16k", "fwd_64k"])
def test_full_step_sampled(hsa, dev, name):
    """The bench's step at its full size and launch configuration (select, forward and
    backward on one workspace with HSA_BWD_AFTER_FWD), on sampled tokens and chunks; the
    selection is compared on every row (the chunk gradients need every selector)."""
    from chunk_sparse_attention_amd import _lib
    wl = workloads.WORKLOADS[name]
    say("case full step", name)
    x = workloads.make_inputs(wl, seed=0)
    Q, K, V, Qs = (x[k].to(dev) for k in ("Q", "K", "V", "Qs"))
    dO = x["dO"].to(dev)
    prob = hsa.problem(wl.B, wl.L, wl.Hq, wl.Hkv, wl.D, wl.K, wl.dtype)
    ws = hsa.workspace(_lib.HSA_OP_BWD, prob, dev)
    Kslc, idx, score, w = hsa.select(Qs, K, wl.K)
    O = hsa.fwd(Q, K, V, idx, w, ws=ws)
    grads = hsa.bwd(Q, K, V, Qs, Kslc, idx, score, w, dO, ws=ws, after_fwd=True)
    torch.cuda.synchronize()
    g = dict(Q=Q, K=K, V=V, Qs=Qs, Kslc=Kslc, idx=idx, score=score, w=w, O=O)
    orc = oracle.get()
    om = None if name == "fwd_16k" else _sample_rows(wl, 384, seed=8)
    f, diff, _ = compare_forward(orc, x, wl, g, out_mask=om)
    tm = _sample_rows(wl, 32, seed=4)
    rng = np.random.default_rng(5)
    cm = np.zeros((wl.B, wl.nC), np.uint8)
    for b in range(wl.B):
        cm[b, rng.choice(wl.nC, size=4, replace=False)] = 1
        cm[b, [0, wl.nC - 1]] = 1
    compare_backward(orc, x, wl, g, f, diff, grads, tok_mask=tm, chunk_mask=cm)


@pytest.mark.parametrize("D,Hq,Hkv,nC", [(64, 8, 2, 16384), (128, 4, 1, 16384),
                                         (64, 4, 1, 16384 + 1500)],
                         ids=["d64", "d128", "d64_two_index_parts"])
def test_max_chunks_step_sampled(hsa, dev, D, Hq, Hkv, nC):
    """Long sequences (16384 chunks, the most the chunk-major forward takes, and 17884, where
    the forward runs on token tiles and the backward's inverse index splits the chunks into
    two parts), each with a ragged tail of 37 tokens: select, forward and backward on one
    workspace.  dO is zero except on a sample T of rows, so that the rows outside T add exact
    zeros to every gradient; the oracle then needs only T's selection (its other rows select
    nothing), and dK, dV, dKslc are compared on the chunks T selected plus others that must
    stay zero, dQ and dQs on T and rows outside it."""
    from chunk_sparse_attention_amd import _lib
    wl = W(f"max_chunks_d{D}_nc{nC}", 1, 64 * nC + 37, Hq, Hkv, D, 64, 8, torch.bfloat16)
    assert wl.G == 4  # the matrix-core forward and backward
    say("case max chunks step", wl)
    x = workloads.make_inputs(wl, seed=11)
    T = _sample_rows(wl, 40, seed=12)
    x["dO"][torch.from_numpy(T == 0)] = 0
    Q, K, V, Qs, dO = (x[k].to(dev) for k in ("Q", "K", "V", "Qs", "dO"))
    prob = hsa.problem(wl.B, wl.L, wl.Hq, wl.Hkv, wl.D, wl.K, wl.dtype)
    ws = hsa.workspace(_lib.HSA_OP_BWD, prob, dev)
    Kslc, idx, score, w = hsa.select(Qs, K, wl.K)
    O = hsa.fwd(Q, K, V, idx, w, ws=ws)
    grads = hsa.bwd(Q, K, V, Qs, Kslc, idx, score, w, dO, ws=ws, after_fwd=True)
    torch.cuda.synchronize()
    g = dict(Q=Q, K=K, V=V, Qs=Qs, Kslc=Kslc, idx=idx, score=score, w=w, O=O)
    del Q, K, V, Qs, dO
    orc = oracle.get()
    f, diff, _ = compare_forward(orc, x, wl, g, row_mask=T)
    rng = np.random.default_rng(13)
    tm = T.copy()
    tm[0, rng.choice(wl.L, size=64, replace=False)] = 1  # rows whose gradients must be zero
    cm = np.zeros((wl.B, wl.nC), np.uint8)
    sel = npy(g["idx"])[T.astype(bool)].astype(np.int64)
    cm[0, np.unique(sel[sel >= 0])] = 1
    picked = int(cm.sum())
    cm[0, rng.choice(wl.nC, size=16, replace=False)] = 1
    cm[0, [0, wl.nC - 1]] = 1
    say("chunks selected by the sample:", picked, "compared:", int(cm.sum()))
    compare_backward(orc, x, wl, g, f, diff, grads, tok_mask=tm, chunk_mask=cm, sel_rows=T)
    tail = slice(wl.nC * wl.S, wl.L)
    assert torch.count_nonzero(grads["dK"][:, tail]).item() == 0
    assert torch.count_nonzero(grads["dV"][:, tail]).item() == 0


def test_full_decode(hsa, dev):
    wl = workloads.WORKLOADS["decode_1m"]
    say("case full decode decode_1m")
    x = workloads.make_decode_inputs(wl, seed=0, slab=1)
    q, qs = x["q"].to(dev), x["qs"].to(dev)
    Kc, Vc = x["Kc"].to(dev), x["Vc"].to(dev)
    Kslc = hsa.pool(Kc)
    O, idx, score, w = hsa.decode(q, qs, Kc, Vc, Kslc, wl.K)
    torch.cuda.synchronize()
    orc = oracle.get()
    ks = orc.pool(x["Kc"], 64)
    assert np.array_equal(npy(Kslc), ks)
    d = orc.decode(x["q"], x["qs"], x["Kc"], x["Vc"], ks, 64, wl.K)
    say("decode idx equal:", bool(np.array_equal(npy(idx), d["idx"])))
    assert np.array_equal(npy(idx), d["idx"])
    assert max_abs(npy(w), d["w"]) <= 1e-5
    assert max_abs(npy(O), d["O"]) <= 2e-2


# ---- the normalisers at the boundary, and the forward state's records ----------------------

LSE_CASES = [w for w in SMALL if w.name in ("tiny_fp32", "bf16_d64_ragged", "bf16_d128_ragged",
                                           "bf16_g1_k3", "bf16_d64_g16_k16", "bf16_g2_d128")]


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "default"])
@pytest.mark.parametrize("wl", LSE_CASES, ids=lambda w: w.name)
def test_lse_out_and_in(hsa, dev, wl, generic):
    """hsa_fwd's optional lse equals the oracle's normaliser log(1 + sum_j exp(z_j)) of every
    (token, head, slot) (0 on masked slots); hsa_bwd given that lse (and no forward state)
    matches the oracle's gradients."""
    say("case lse", wl, generic)
    orc = oracle.get()
    x = workloads.make_inputs(wl, seed=12)
    Q, K, V, Qs, dO = (x[k].to(dev) for k in ("Q", "K", "V", "Qs", "dO"))
    Kslc, idx, score, w = hsa.select(Qs, K, wl.K, generic=generic)
    O, lse = hsa.fwd(Q, K, V, idx, w, generic=generic, want_lse=True)
    grads = hsa.bwd(Q, K, V, Qs, Kslc, idx, score, w, dO, generic=generic, lse=lse)
    torch.cuda.synchronize()
    gi, gw = npy(idx).astype(np.int32), npy(w)
    Oo, lo = orc.attend(x["Q"], x["K"], x["V"], gi, gw, wl.S, want_lse=True)
    assert max_abs(npy(O), Oo) <= tol_for(wl.dtype)
    valid = np.repeat(gi >= 0, wl.G, axis=2)  # [B, L, Hq, K]
    gl = npy(lse)
    assert np.all(gl[~valid] == 0)
    err = max_abs(gl, lo)
    say("lse max abs", err)
    assert err <= (1e-4 if wl.dtype == torch.float32 else 1e-3), err
    g = dict(Q=Q, K=K, V=V, Qs=Qs, Kslc=Kslc, idx=idx, score=score, w=w, O=O)
    f, diff, _ = compare_forward(orc, x, wl, g)
    compare_backward(orc, x, wl, g, f, diff, grads)


def _invidx_launches(hsa, fn):
    hsa.timer_enable(True)
    out = fn()
    torch.cuda.synchronize()
    n = hsa.timer_read()["invidx"][0]
    hsa.timer_enable(False)
    return out, n


def test_after_fwd_stale_workspace(hsa, dev):
    """HSA_BWD_AFTER_FWD reuses the forward's state only when the library's record of the
    workspace names the same problem, Q, K, idx and w: after a forward of another selection
    on the workspace, or a backward of another problem that rebuilt it, the flagged backward
    rebuilds its index (one index launch instead of none) and equals, bit for bit, the
    backward without the flag, and the oracle."""
    from chunk_sparse_attention_amd import _lib
    wl = SMALL[1]  # bf16_d64_ragged: the chunk-major forward and the matrix-core backward
    say("case stale workspace", wl)
    orc = oracle.get()
    x = workloads.make_inputs(wl, seed=14)
    Q, K, V, Qs, dO = (x[k].to(dev) for k in ("Q", "K", "V", "Qs", "dO"))
    Kslc, idx, score, w = hsa.select(Qs, K, wl.K)
    other = workloads.make_selection(wl.B, wl.L, wl.Hkv, wl.S, wl.K, seed=15)
    idx2, w2 = other["idx"].to(dev), other["w"].to(dev)
    prob = hsa.problem(wl.B, wl.L, wl.Hq, wl.Hkv, wl.D, wl.K, wl.dtype)
    ws = hsa.workspace(_lib.HSA_OP_BWD, prob, dev)
    alone = hsa.bwd(Q, K, V, Qs, Kslc, idx, score, w, dO)

    def flagged():
        return hsa.bwd(Q, K, V, Qs, Kslc, idx, score, w, dO, ws=ws, after_fwd=True)

    # 1. the matching forward: the state is reused (no index launch)
    O = hsa.fwd(Q, K, V, idx, w, ws=ws)
    fresh, n = _invidx_launches(hsa, flagged)
    assert n == 0, n
    # 2. a forward of another selection on the same workspace: rebuilt
    hsa.fwd(Q, K, V, idx2, w2, ws=ws)
    stale, n = _invidx_launches(hsa, flagged)
    assert n == 1, n
    for k in ("dQ", "dK", "dV", "dQs", "dKslc"):
        assert torch.equal(stale[k], alone[k]), k
    # 3. the matching forward, then a backward of another problem (smaller K) without the
    #    flag on the same workspace, which rebuilds the index there: rebuilt again
    hsa.fwd(Q, K, V, idx, w, ws=ws)
    small = hsa.bwd(Q, K, V, Qs, Kslc, idx[..., :4].contiguous(), score[..., :4].contiguous(),
                    w[..., :4].contiguous(), dO, ws=ws)
    stale2, n = _invidx_launches(hsa, flagged)
    assert n == 1, n
    for k in ("dQ", "dK", "dV", "dQs", "dKslc"):
        assert torch.equal(stale2[k], alone[k]), k
    # 4. no forward ever ran on a fresh workspace: rebuilt
    ws3 = hsa.workspace(_lib.HSA_OP_BWD, prob, dev)
    never = hsa.bwd(Q, K, V, Qs, Kslc, idx, score, w, dO, ws=ws3, after_fwd=True)
    torch.cuda.synchronize()
    for k in ("dQ", "dK", "dV", "dQs", "dKslc"):
        assert torch.equal(never[k], alone[k]), k
    del small
    g = dict(Q=Q, K=K, V=V, Qs=Qs, Kslc=Kslc, idx=idx, score=score, w=w, O=O)
    f, diff, _ = compare_forward(orc, x, wl, g)
    compare_backward(orc, x, wl, g, f, diff, stale)
    compare_backward(orc, x, wl, g, f, diff, fresh)


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "default"])
def test_repeated_chunks_in_a_row(hsa, dev, generic):
    """A caller's selection that repeats a chunk within a row (outside hsa_fwd's contract, and
    never produced by hsa_select): up to 16384 chunks every repeated slot still adds its own
    term, as in the oracle, and the backward differentiates each slot; the inverse index
    gives the repeated slots their own entries."""
    wl = SMALL[1]
    say("case repeated chunks", generic)
    orc = oracle.get()
    x = workloads.make_inputs(wl, seed=16)
    sel = workloads.make_selection(wl.B, wl.L, wl.Hkv, wl.S, wl.K, seed=17)
    idx = sel["idx"].clone()
    rows = torch.arange(3 * 64, wl.L, 7)
    idx[0, rows, 0, 1] = idx[0, rows, 0, 0]           # slot 1 repeats slot 0
    idx[1, rows, 1, 3] = idx[1, rows, 1, 2]           # slot 3 repeats slot 2
    idx[1, rows[::3], 0, 2] = idx[1, rows[::3], 0, 0]  # slots 0 and 2 agree
    Q, K, V, Qs, dO = (x[k].to(dev) for k in ("Q", "K", "V", "Qs", "dO"))
    d_idx, score, w = idx.to(dev), sel["score"].to(dev), sel["w"].to(dev)
    Kslc = hsa.pool(K)
    O = hsa.fwd(Q, K, V, d_idx, w, generic=generic)
    grads = hsa.bwd(Q, K, V, Qs, Kslc, d_idx, score, w, dO, generic=generic)
    torch.cuda.synchronize()
    tol = tol_for(wl.dtype)
    Oo = orc.attend(x["Q"], x["K"], x["V"], idx, sel["w"], wl.S)
    assert max_abs(npy(O), Oo) <= tol
    o = orc.backward(x["Q"], x["K"], x["V"], x["Qs"], orc.pool(x["K"], wl.S), idx,
                     sel["score"], sel["w"], x["dO"], wl.S)
    rep = {k: max_abs(npy(grads[k]), o[k]) for k in ("dQ", "dK", "dV", "dQs", "dKslc")}
    say("repeated chunks", rep)
    for k, v in rep.items():
        assert v <= tol, (k, v)
