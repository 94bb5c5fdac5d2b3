"""Pins that tie the CPU oracle to what the pages and the mathematics fix.

Each ``pin_*`` takes an oracle handle and raises AssertionError when the oracle disagrees
with something other than itself: a library routine (torch's bf16 cast, scaled dot-product
attention, autograd), a closed form, an invariant, a brute-force dense formulation, or
finite differences of the oracle's own forward.  ``test_oracle_pins.py`` runs every pin on
the oracle; ``test_oracle_mutations.py`` runs them on builds with one planted mistake each
and requires that some pin fails.

Sources: "Hardware-aligned Hierarchical Sparse Attention for Efficient Long-term Memory
Access", papernotes.org note, section 方法详解 › 层次化稀疏注意力（HSA） (chunk selection by
mean-pooled keys, per query group; token-level attention per chunk; stick-breaking fusion on
the sigmoid of the scores), › 硬件对齐 Kernel (softmax-off-by-one; two-phase backward), ›
训练与推理优化 (decode against the resident chunk table).
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle as O
import workloads

F32, BF16, F64 = O.F32, O.BF16, O.F64


def _rand(gen, shape, std=1.0, dtype=torch.float64):
    return (torch.randn(shape, generator=gen, dtype=torch.float64) * std).to(dtype)


# ----------------------------------------------------------------------------------------
# rounding (the storage step of the chunk key)
# ----------------------------------------------------------------------------------------
def pin_round_matches_torch(orc):
    """bf16 / fp32 rounding equals torch's own float32->bfloat16 and float64->float32 casts
    (both round to nearest, ties to even) on values exactly representable in fp32,
    including exact ties, subnormals and values near overflow."""
    gen = torch.Generator().manual_seed(1)
    x = torch.randn(4000, generator=gen, dtype=torch.float32) * 3
    extra = torch.tensor([0.0, -0.0, 1.0, 1.00390625, 1.01171875, -1.00390625, 3.0e38, -3.3e38,
                          1e-40, -1e-39, 1.1754944e-38, 2.0 ** -130, 2.0 ** -133 * 3,
                          255.5, 256.5, 257.0], dtype=torch.float32)
    tie = torch.arange(1, 200, dtype=torch.float32)
    x = torch.cat([x, extra, 1.0 + tie * 2.0 ** -8, -(1.0 + tie * 2.0 ** -8)])
    ref = x.to(torch.bfloat16).to(torch.float64)
    got = torch.tensor([orc.round(float(v), BF16) for v in x.tolist()], dtype=torch.float64)
    assert torch.equal(got, ref), (x[got != ref][:5], got[got != ref][:5], ref[got != ref][:5])
    y = torch.randn(2000, generator=gen, dtype=torch.float64) * 1e3
    ref32 = y.to(torch.float32).to(torch.float64)
    got32 = torch.tensor([orc.round(float(v), F32) for v in y.tolist()], dtype=torch.float64)
    assert torch.equal(got32, ref32)


# ----------------------------------------------------------------------------------------
# F1 pooling
# ----------------------------------------------------------------------------------------
def pin_pool_closed_forms(orc):
    """Constant chunks pool to that row exactly; a chunk whose rows are r*u pools to
    mean(r)*u; any chunk pools to torch's float64 mean rounded by torch's bf16 cast."""
    S, D = 16, 8
    gen = torch.Generator().manual_seed(2)
    row = _rand(gen, (D,), dtype=torch.float32)
    K = row.expand(1, 3 * S, 1, D).contiguous()
    ks = orc.pool(K, S)
    assert np.array_equal(ks, np.broadcast_to(row.double().numpy(), ks.shape))
    u = torch.tensor([1.0, -2.0, 0.5, 4.0, 0.25, -8.0, 1.5, 3.0], dtype=torch.float32)
    r = torch.arange(S, dtype=torch.float32)  # mean = (S-1)/2
    K2 = (r[:, None] * u[None, :]).reshape(1, S, 1, D)
    ks2 = orc.pool(K2, S)
    assert np.allclose(ks2[0, 0, 0], ((S - 1) / 2.0) * u.double().numpy(), rtol=0, atol=1e-12)
    K3 = _rand(gen, (2, 5 * S, 3, D), 0.5, torch.float32).to(torch.bfloat16)
    ks3 = orc.pool(K3, S)
    ref = K3.double().reshape(2, 5, S, 3, D).mean(2).to(torch.float32).to(torch.bfloat16)
    # double -> f32 -> bf16 can double-round; compare against the single rounding directly
    ref_single = torch.tensor([orc.round(v, BF16) for v in
                               K3.double().reshape(2, 5, S, 3, D).mean(2).flatten().tolist()])
    assert np.array_equal(ks3.reshape(-1), ref_single.numpy())
    assert np.abs(ks3 - ref.double().numpy()).max() <= 2.0 ** -8 * np.abs(ks3).max()


# ----------------------------------------------------------------------------------------
# F2-F4 selection and weights
# ----------------------------------------------------------------------------------------
def _brute_select(Qs, Kslc, S, K, sel_scale):
    """Full sort of every causal candidate with numpy (lexsort: score desc, index asc)."""
    Qs = Qs.double().numpy()
    B, L, Hkv, D = Qs.shape
    nC = Kslc.shape[1]
    idx = np.full((B, L, Hkv, K), -1, np.int32)
    sc = np.full((B, L, Hkv, K), -np.inf)
    for b in range(B):
        for g in range(Hkv):
            s_all = (Qs[b, :, g, :] @ Kslc[b, :, g, :].T) * sel_scale  # [L, nC]
            s_all = s_all.astype(np.float32).astype(np.float64)
            for t in range(L):
                n = min(t // S, nC)
                if n == 0:
                    continue
                s = s_all[t, :n]
                order = np.lexsort((np.arange(n), -s))[:K]
                idx[b, t, g, :len(order)] = order
                sc[b, t, g, :len(order)] = s[order]
    return idx, sc


def pin_select_bruteforce(orc):
    """Selection equals a full numpy sort of all causal candidates (bf16 and fp32 inputs)."""
    gen = torch.Generator().manual_seed(3)
    for dt, S, K in ((torch.bfloat16, 16, 3), (torch.float32, 8, 5)):
        B, L, Hkv, D = 2, 12 * S + 5, 2, 16
        Kmat = _rand(gen, (B, L, Hkv, D), 0.5, torch.float32).to(dt)
        Qs = _rand(gen, (B, L, Hkv, D), 1.0, torch.float32).to(dt)
        ks = orc.pool(Kmat, S)
        sel = 1.0 / math.sqrt(D)
        idx, score, w = orc.select(Qs, ks, S, K, sel)
        bidx, bsc = _brute_select(Qs, ks, S, K, sel)
        assert np.array_equal(idx, bidx)
        assert np.array_equal(score, bsc)


def pin_select_ties_and_causality(orc):
    """Qs = 0 makes every score 0: the tie rule then picks chunks 0..K-1 in order and
    stick-breaking gives w_k = 2^-(k+1).  Tokens t < S have no chunk; tokens in [S, 2S) have
    exactly chunk 0; duplicate chunk keys rank the lower index first."""
    S, K, D = 8, 4, 8
    gen = torch.Generator().manual_seed(4)
    L = 10 * S
    Kmat = _rand(gen, (1, L, 1, D), 0.5, torch.float32)
    Qs = torch.zeros((1, L, 1, D), dtype=torch.float32)
    ks = orc.pool(Kmat, S)
    idx, score, w = orc.select(Qs, ks, S, K)
    for t in range(L):
        n = min(t // S, K)
        assert list(idx[0, t, 0]) == list(range(n)) + [-1] * (K - n), (t, idx[0, t, 0])
        assert np.allclose(w[0, t, 0, :n], [2.0 ** -(k + 1) for k in range(n)], rtol=0,
                           atol=1e-15)
        assert np.all(w[0, t, 0, n:] == 0) and np.all(np.isneginf(score[0, t, 0, n:]))
    # duplicate chunks: chunks 2 and 5 share their keys and are the best match
    Kd = _rand(gen, (1, L, 1, D), 0.1, torch.float32)
    v = torch.tensor([3.0] * D)
    Kd[0, 2 * S:3 * S, 0, :] = v
    Kd[0, 5 * S:6 * S, 0, :] = v
    Qd = torch.ones((1, L, 1, D), dtype=torch.float32)
    idx, score, w = orc.select(Qd, orc.pool(Kd, S), S, K)
    for t in range(6 * S, L):
        assert idx[0, t, 0, 0] == 2 and idx[0, t, 0, 1] == 5, idx[0, t, 0]


def pin_select_nonfinite_and_signed_zero(orc):
    """The ranking rule on values that are not ordinary numbers: a NaN score ranks as -inf
    (last, ties among such chunks to the lower index, weight 0); +inf and -inf rank as the
    extremes they are (an +inf slot takes all of the remaining stick); -0 ranks equal to +0,
    so a row whose scores all round to a signed zero keeps chunk index order.  Checked
    against a brute-force sort that applies exactly that rule to scores computed with numpy.
    Inputs are small dyadic integers and the scale a power of two, so every finite score is
    exact whatever the summation order and the comparison can demand equality."""
    gen = torch.Generator().manual_seed(31)
    S, K, D, Hkv = 4, 3, 8, 2
    L = 12 * S + 2
    nC = L // S
    Kmat = torch.randint(-4, 5, (1, L, Hkv, D), generator=gen).to(torch.float32) * 0.25
    Qs = torch.randint(-3, 4, (1, L, Hkv, D), generator=gen).to(torch.float32)
    nan, inf = float("nan"), float("inf")
    Qs[0, 17, 0, :] = nan           # every score NaN: chunks in index order, weight 0
    Qs[0, 21, 1, 2] = nan           # one NaN component: same
    Qs[0, 23, 1, 0] = inf           # scores +inf, -inf or NaN (0 * inf) by the key's sign
    Qs[0, 30, 0, 5] = -inf
    Kmat[0, 3 * S + 1, 0, 4] = nan  # chunk 3 of group 0: NaN for every token of group 0
    Kmat[0, 5 * S + 2, 1, 6] = inf  # chunk 5 of group 1: +-inf or NaN scores
    tiny = 2.0 ** -140              # rows whose every score rounds to a signed zero in fp32
    Qs[0, 38, 1, :] = torch.tensor([tiny, -tiny, tiny, 0, 0, 0, 0, 0])
    Qs[0, 41, 0, :] = -tiny
    sel = 2.0 ** -20
    ks = orc.pool(Kmat, S)
    idx, score, w = orc.select(Qs, ks, S, K, sel)

    q = Qs.double().numpy()
    ref_idx = np.full((1, L, Hkv, K), -1, np.int32)
    ref_sc = np.full((1, L, Hkv, K), -np.inf)
    for g in range(Hkv):
        with np.errstate(invalid="ignore", over="ignore"):
            s_all = (q[0, :, g, :] @ ks[0, :, g, :].T) * sel
        s_all = s_all.astype(np.float32).astype(np.float64)
        s_all[np.isnan(s_all)] = -np.inf   # the rule: NaN ranks as -inf
        s_all[s_all == 0] = 0.0            # the rule: -0 ranks as +0
        for t in range(L):
            n = min(t // S, nC)
            if n == 0:
                continue
            s = s_all[t, :n]
            order = np.lexsort((np.arange(n), -s))[:K]
            ref_idx[0, t, g, :len(order)] = order
            ref_sc[0, t, g, :len(order)] = s[order]
    assert np.array_equal(idx, ref_idx), np.argwhere(idx != ref_idx)[:5]
    assert not np.isnan(score).any() and not np.isnan(w).any()
    assert np.array_equal(score, ref_sc), np.argwhere(score != ref_sc)[:5]
    # the planted rows do what the rule says
    assert list(idx[0, 17, 0]) == [0, 1, 2] and np.all(np.isneginf(score[0, 17, 0]))
    assert np.all(w[0, 17, 0] == 0) and np.all(w[0, 21, 1] == 0)
    assert list(idx[0, 38, 1]) == [0, 1, 2] and list(idx[0, 41, 0]) == [0, 1, 2]
    assert np.all(score[0, 38, 1] == 0) and np.all(score[0, 41, 0] == 0)
    assert 3 not in idx[0, 4 * S:, 0, :2]  # chunk 3 of group 0 never beats a finite score
    row = score[0, 23, 1]
    assert np.isposinf(row[0]) and w[0, 23, 1, 0] == 1.0 and np.all(w[0, 23, 1, 1:] == 0)
    # stick-breaking on the other rows is untouched by the rule
    valid = np.isfinite(score)
    p = 1.0 / (1.0 + np.exp(-np.where(valid, score, 0.0)))
    assert np.allclose(w[..., 0][valid[..., 0]], p[..., 0][valid[..., 0]], rtol=1e-14, atol=0)


def pin_stick_breaking_identities(orc):
    """For any scores: w >= 0, w_0 = sigmoid(s_0), and sum_k w_k = 1 - prod_k (1 - sigmoid(s_k))
    (the telescoping identity of stick-breaking), so sum_k w_k <= 1."""
    gen = torch.Generator().manual_seed(5)
    S, K, D = 8, 6, 16
    L = 12 * S
    Kmat = _rand(gen, (2, L, 2, D), 1.0, torch.float32)
    Qs = _rand(gen, (2, L, 2, D), 3.0, torch.float32)
    idx, score, w = orc.select(Qs, orc.pool(Kmat, S), S, K)
    valid = idx >= 0
    p = np.where(valid, 1.0 / (1.0 + np.exp(-np.where(valid, score, 0.0))), 0.0)
    assert np.all(w >= 0)
    assert np.allclose(w[..., 0][valid[..., 0]], p[..., 0][valid[..., 0]], rtol=1e-14, atol=0)
    total = 1.0 - np.prod(1.0 - p, axis=-1)
    assert np.allclose(w.sum(-1), total, rtol=1e-12, atol=1e-15)
    assert np.all(w.sum(-1) <= 1.0 + 1e-15)
    # scaling Qs by a positive factor keeps the ranking (and so idx)
    idx2, _, _ = orc.select(Qs * 2.0, orc.pool(Kmat, S), S, K)
    assert np.array_equal(idx, idx2)


def pin_softmax_weights_identities(orc):
    """The softmax variant of the chunk weights: the same selection as stick-breaking, every
    row's valid weights positive and summing to 1, and closed forms: Qs = 0 gives each of a
    row's n valid slots 1/n; K = 1 gives weight 1."""
    gen = torch.Generator().manual_seed(21)
    S, K, D = 8, 6, 16
    L = 12 * S
    Kmat = _rand(gen, (2, L, 2, D), 1.0, torch.float32)
    Qs = _rand(gen, (2, L, 2, D), 3.0, torch.float32)
    ks = orc.pool(Kmat, S)
    idx, score, w = orc.select(Qs, ks, S, K, weights="softmax")
    idx_sb, _, _ = orc.select(Qs, ks, S, K)
    assert np.array_equal(idx, idx_sb)
    valid = idx >= 0
    assert np.all(w[valid] > 0) and np.all(w[~valid] == 0)
    rows = valid.any(-1)
    assert np.allclose(w.sum(-1)[rows], 1.0, rtol=0, atol=1e-14)
    # the log-weights of a row differ by the score differences (base e, increasing in s)
    both = valid[..., 1:] & valid[..., :1]
    dlog = np.log(np.where(valid, w, 1.0))
    sv = np.where(valid, score, 0.0)
    gap = (dlog[..., 1:] - dlog[..., :1]) - (sv[..., 1:] - sv[..., :1])
    assert np.allclose(np.where(both, gap, 0.0), 0.0, rtol=0, atol=1e-12)
    assert np.all(w.sum(-1)[~rows] == 0)
    # Qs = 0: every score 0, uniform weights over the n_avail = min(K, t // S) slots
    _, _, w0 = orc.select(torch.zeros_like(Qs), ks, S, K, weights="softmax")
    for t in range(L):
        n = min(K, t // S)
        expect = np.array([1.0 / n] * n + [0.0] * (K - n)) if n else np.zeros(K)
        assert np.allclose(w0[:, t], expect, rtol=0, atol=1e-15), t
    # K = 1: the single slot takes all the weight
    idx1, _, w1 = orc.select(Qs, ks, S, 1, weights="softmax")
    assert np.all(w1[idx1 >= 0] == 1.0) and np.all(w1[idx1 < 0] == 0.0)


# ----------------------------------------------------------------------------------------
# F5-F6 attention
# ----------------------------------------------------------------------------------------
def pin_softmax1_equals_sdpa(orc):
    """With one selected chunk of weight 1, each head's output equals torch's scaled
    dot-product attention over the chunk's S keys plus one appended zero key whose value row
    is zero (that extra logit is the 'off-by-one')."""
    gen = torch.Generator().manual_seed(6)
    S, D, Hq, Hkv = 16, 8, 4, 2
    L = 4 * S
    Q = _rand(gen, (1, L, Hq, D), 1.5, torch.float32)
    Km = _rand(gen, (1, L, Hkv, D), 1.5, torch.float32)
    V = _rand(gen, (1, L, Hkv, D), 1.0, torch.float32)
    idx = torch.full((1, L, Hkv, 1), -1, dtype=torch.int32)
    c_of = [(t // S) - 1 if t >= S else -1 for t in range(L)]
    for t in range(L):
        idx[0, t, :, 0] = c_of[t]
    w = (idx >= 0).double()
    scale = 0.37
    out = orc.attend(Q, Km, V, idx, w, S, sm_scale=scale)
    G = Hq // Hkv
    for t in range(S, L):
        c = c_of[t]
        for h in range(Hq):
            g = h // G
            kk = torch.cat([Km[0, c * S:(c + 1) * S, g].double(), torch.zeros(1, D, dtype=torch.float64)])
            vv = torch.cat([V[0, c * S:(c + 1) * S, g].double(), torch.zeros(1, D, dtype=torch.float64)])
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q[0, t, h].double()[None, None, None], kk[None, None], vv[None, None], scale=scale)
            assert np.allclose(out[0, t, h], ref.reshape(-1).numpy(), rtol=1e-12, atol=1e-13)
    assert np.all(out[0, :S] == 0)


def pin_lse_equals_logsumexp(orc):
    """The normaliser the oracle reports for every (token, head, slot) is torch's logsumexp
    over the chunk's S scaled logits plus one zero logit; Q = 0 gives log(S + 1) exactly; a
    masked slot reports 0."""
    gen = torch.Generator().manual_seed(16)
    S, D, Hq, Hkv, K = 8, 8, 4, 2, 3
    L = 6 * S + 3
    Q = _rand(gen, (1, L, Hq, D), 2.0, torch.float32)
    Km = _rand(gen, (1, L, Hkv, D), 2.0, torch.float32)
    V = _rand(gen, (1, L, Hkv, D), 1.0, torch.float32)
    sel = workloads.make_selection(1, L, Hkv, S, K, seed=17)
    sm = 0.45
    _, lse = orc.attend(Q, Km, V, sel["idx"], sel["w"], S, sm_scale=sm, want_lse=True)
    G = Hq // Hkv
    idx = np.asarray(sel["idx"])
    for t in range(L):
        for h in range(Hq):
            for k in range(K):
                c = int(idx[0, t, h // G, k])
                if c < 0:
                    assert lse[0, t, h, k] == 0.0
                    continue
                z = (Km[0, c * S:(c + 1) * S, h // G].double() @ Q[0, t, h].double()) * sm
                ref = torch.logsumexp(torch.cat([z, torch.zeros(1, dtype=torch.float64)]), 0)
                assert abs(lse[0, t, h, k] - float(ref)) <= 1e-13 * max(1.0, abs(float(ref)))
    _, lse0 = orc.attend(torch.zeros_like(Q), Km, V, sel["idx"], sel["w"], S, want_lse=True)
    valid = np.repeat(idx >= 0, G, axis=2)
    assert np.all(lse0[valid] == math.log(S + 1.0)) and np.all(lse0[~valid] == 0.0)


def pin_zero_query_closed_form(orc):
    """Q = 0 gives every key the same logit 0, so a_j = 1/(S+1) and each chunk contributes
    (S/(S+1)) * mean of its value rows; with weights w the output is their w-weighted sum."""
    gen = torch.Generator().manual_seed(7)
    S, D, K = 16, 8, 3
    L = 6 * S
    Q = torch.zeros((1, L, 2, D), dtype=torch.float32)
    Km = _rand(gen, (1, L, 1, D), 1.0, torch.float32)
    V = _rand(gen, (1, L, 1, D), 1.0, torch.float32)
    sel = workloads.make_selection(1, L, 1, S, K, seed=11)
    out = orc.attend(Q, Km, V, sel["idx"], sel["w"], S)
    Vd = V.double().numpy()
    for t in range(L):
        ref = np.zeros(D)
        for k in range(K):
            c = int(sel["idx"][0, t, 0, k])
            if c >= 0:
                ref += float(sel["w"][0, t, 0, k]) * (S / (S + 1.0)) * Vd[0, c * S:(c + 1) * S, 0].mean(0)
        assert np.allclose(out[0, t, 0], ref, rtol=1e-12, atol=1e-14)
        assert np.allclose(out[0, t, 1], ref, rtol=1e-12, atol=1e-14)


def dense_forward(Q, Km, V, idx, w, S, sm_scale):
    """Brute-force dense formulation (float64 torch): build the full L x L attention matrix
    A[b,h,t,m] = w_k * a_j for key m = c_k*S + j of every selected chunk, where a is torch's
    softmax over the chunk's S logits plus one zero logit; then O = A @ V."""
    B, L, Hq, D = Q.shape
    Hkv = Km.shape[2]
    G = Hq // Hkv
    Kt = idx.shape[-1]
    Kh = Km.repeat_interleave(G, dim=2)  # [B, L, Hq, D]
    Vh = V.repeat_interleave(G, dim=2)
    logits = torch.matmul(Q.permute(0, 2, 1, 3), Kh.permute(0, 2, 3, 1).contiguous()) * sm_scale
    A = torch.zeros((B, Hq, L, L), dtype=torch.float64)
    idx_h = idx.long().repeat_interleave(G, dim=2)  # [B, L, Hq, K]
    w_h = w.repeat_interleave(G, dim=2)
    for b in range(B):
        for h in range(Hq):
            for t in range(L):
                for k in range(Kt):
                    c = int(idx_h[b, t, h, k])
                    if c < 0:
                        continue
                    z = torch.cat([logits[b, h, t, c * S:(c + 1) * S],
                                   torch.zeros(1, dtype=torch.float64)])
                    a = torch.softmax(z, dim=0)[:S]
                    A[b, h, t, c * S:(c + 1) * S] = A[b, h, t, c * S:(c + 1) * S] + w_h[b, t, h, k] * a
    return torch.matmul(A, Vh.permute(0, 2, 1, 3)).permute(0, 2, 1, 3)


def pin_dense_bruteforce(orc):
    """Oracle attention equals the dense L x L formulation on random inputs and selections,
    and is linear in V."""
    gen = torch.Generator().manual_seed(8)
    B, S, Hq, Hkv, D, K = 2, 8, 4, 2, 8, 3
    L = 7 * S + 3
    Q = _rand(gen, (B, L, Hq, D), 1.0)
    Km = _rand(gen, (B, L, Hkv, D), 1.0)
    V = _rand(gen, (B, L, Hkv, D), 1.0)
    sel = workloads.make_selection(B, L, Hkv, S, K, seed=12)
    sm = 0.3
    got = orc.attend(Q, Km, V, sel["idx"], sel["w"], S, sm_scale=sm)
    ref = dense_forward(Q, Km, V, sel["idx"], sel["w"].double(), S, sm)
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-13)
    V2 = _rand(gen, (B, L, Hkv, D), 1.0)
    lin = orc.attend(Q, Km, V + 2.0 * V2, sel["idx"], sel["w"], S, sm_scale=sm)
    parts = got + 2.0 * orc.attend(Q, Km, V2, sel["idx"], sel["w"], S, sm_scale=sm)
    assert np.allclose(lin, parts, rtol=1e-12, atol=1e-12)


def pin_permutation_within_chunk(orc):
    """Permuting the rows of a past chunk (its keys and values together) leaves every later
    output unchanged (attention inside a chunk has no positional term)."""
    gen = torch.Generator().manual_seed(9)
    S, D, K = 8, 8, 2
    L = 8 * S
    Q = _rand(gen, (1, L, 2, D), 1.0, torch.float32)
    Km = _rand(gen, (1, L, 1, D), 1.0, torch.float32)
    V = _rand(gen, (1, L, 1, D), 1.0, torch.float32)
    Qs = _rand(gen, (1, L, 1, D), 1.0, torch.float32)
    base = orc.forward(Q, Km, V, Qs, S, K)
    perm = torch.randperm(S, generator=gen)
    Kp, Vp = Km.clone(), V.clone()
    Kp[0, 2 * S:3 * S] = Km[0, 2 * S + perm]
    Vp[0, 2 * S:3 * S] = V[0, 2 * S + perm]
    got = orc.forward(Q, Kp, Vp, Qs, S, K)
    assert np.array_equal(base["idx"], got["idx"])
    assert np.allclose(base["O"], got["O"], rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------------------
# B1-B5 backward
# ----------------------------------------------------------------------------------------
def _loss_and_grads(orc, Q, Km, V, Qs, dO, S, K, sm, sel, weights="stick"):
    f = orc.forward(Q, Km, V, Qs, S, K, sm_scale=sm, sel_scale=sel, score_dt=F64,
                    weights=weights)
    loss = float((f["O"] * dO.numpy()).sum())
    return f, loss


def pin_backward_finite_differences(orc):
    """The hand-derived backward equals central finite differences of the oracle's own
    forward (pool -> select -> attend, in float64 with no score rounding), for directional
    derivatives along random directions in Q, K, V and Qs.  The chosen inputs have no
    near-ties, so the ranking is constant over the step."""
    _finite_differences(orc, "stick", 10)


def pin_backward_finite_differences_softmax(orc):
    """The same check with the softmax chunk weights: it pins their chain rule into the
    selection scores (and so dQs and the pooled-key gradient)."""
    _finite_differences(orc, "softmax", 11)


def _finite_differences(orc, weights, seed):
    gen = torch.Generator().manual_seed(seed)
    B, S, Hq, Hkv, D, K = 1, 8, 4, 2, 8, 3
    L = 7 * S
    Q = _rand(gen, (B, L, Hq, D), 1.0)
    Km = _rand(gen, (B, L, Hkv, D), 1.0)
    V = _rand(gen, (B, L, Hkv, D), 1.0)
    Qs = _rand(gen, (B, L, Hkv, D), 2.0)
    dO = _rand(gen, (B, L, Hq, D), 1.0)
    sm, sel = 0.35, 0.5
    f, _ = _loss_and_grads(orc, Q, Km, V, Qs, dO, S, K, sm, sel, weights)
    g = orc.backward(Q, Km, V, Qs, f["Kslc"], f["idx"], f["score"], f["w"], dO, S, sm, sel,
                     fold=True, weights=weights)
    eps = 1e-6
    for name in ("Q", "K", "V", "Qs"):
        for trial in range(3):
            args = dict(Q=Q, K=Km, V=V, Qs=Qs)
            d = _rand(gen, args[name].shape, 1.0)
            plus = dict(args)
            minus = dict(args)
            plus[name] = args[name] + eps * d
            minus[name] = args[name] - eps * d
            fp, lp = _loss_and_grads(orc, plus["Q"], plus["K"], plus["V"], plus["Qs"], dO, S, K,
                                     sm, sel, weights)
            fm, lm = _loss_and_grads(orc, minus["Q"], minus["K"], minus["V"], minus["Qs"], dO, S,
                                     K, sm, sel, weights)
            assert np.array_equal(fp["idx"], f["idx"]) and np.array_equal(fm["idx"], f["idx"])
            fd = (lp - lm) / (2 * eps)
            grad = {"Q": g["dQ"], "K": g["dK"], "V": g["dV"], "Qs": g["dQs"]}[name]
            an = float((grad * d.numpy()).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, trial, fd, an)


def pin_backward_autograd(orc):
    """The backward equals torch autograd through the dense formulation, with the selection
    held fixed and the weights computed from the scores by stick-breaking; this also checks
    the pooled-key gradient folded into dK and reported as dKslc."""
    gen = torch.Generator().manual_seed(13)
    B, S, Hq, Hkv, D, K = 2, 8, 4, 2, 8, 3
    L = 6 * S + 5
    Q = _rand(gen, (B, L, Hq, D), 1.0)
    Km = _rand(gen, (B, L, Hkv, D), 1.0)
    V = _rand(gen, (B, L, Hkv, D), 1.0)
    Qs = _rand(gen, (B, L, Hkv, D), 2.0)
    dO = _rand(gen, (B, L, Hq, D), 1.0)
    sm, sel = 0.4, 0.3
    f = orc.forward(Q, Km, V, Qs, S, K, sm_scale=sm, sel_scale=sel, score_dt=F64)
    idx = torch.from_numpy(f["idx"])
    g = orc.backward(Q, Km, V, Qs, f["Kslc"], f["idx"], f["score"], f["w"], dO, S, sm, sel,
                     fold=True)
    Qr, Kr, Vr, Qsr = (x.clone().requires_grad_(True) for x in (Q, Km, V, Qs))
    nC = L // S
    Kslc = Kr[:, :nC * S].reshape(B, nC, S, Hkv, D).mean(2)
    valid = idx >= 0
    ic = idx.clamp(min=0).long()
    ks_sel = torch.gather(Kslc.unsqueeze(1).expand(B, L, nC, Hkv, D), 2,
                          ic.permute(0, 1, 3, 2)[..., None].expand(B, L, K, Hkv, D))
    s = sel * (Qsr.unsqueeze(2) * ks_sel).sum(-1).permute(0, 1, 3, 2)  # [B, L, Hkv, K]
    p = torch.where(valid, torch.sigmoid(s), torch.zeros_like(s))
    keep = torch.cumprod(torch.cat([torch.ones_like(p[..., :1]), 1 - p[..., :-1]], -1), -1)
    w = p * keep
    out = dense_forward(Qr, Kr, Vr, idx, w, S, sm)
    (out * dO).sum().backward()
    for name, ref in (("dQ", Qr.grad), ("dK", Kr.grad), ("dV", Vr.grad), ("dQs", Qsr.grad)):
        assert np.allclose(g[name], ref.numpy(), rtol=1e-10, atol=1e-11), name
    # dKslc alone: gradient with Kslc a free leaf
    Kl = Kslc.detach().clone().requires_grad_(True)
    ks_sel = torch.gather(Kl.unsqueeze(1).expand(B, L, nC, Hkv, D), 2,
                          ic.permute(0, 1, 3, 2)[..., None].expand(B, L, K, Hkv, D))
    s = sel * (Qs.unsqueeze(2) * ks_sel).sum(-1).permute(0, 1, 3, 2)
    p = torch.where(valid, torch.sigmoid(s), torch.zeros_like(s))
    keep = torch.cumprod(torch.cat([torch.ones_like(p[..., :1]), 1 - p[..., :-1]], -1), -1)
    out = dense_forward(Q, Km, V, idx, p * keep, S, sm)
    (out * dO).sum().backward()
    assert np.allclose(g["dKslc"], Kl.grad.numpy(), rtol=1e-10, atol=1e-11)
    g2 = orc.backward(Q, Km, V, Qs, f["Kslc"], f["idx"], f["score"], f["w"], dO, S, sm, sel,
                      fold=False)
    diff = g["dK"] - g2["dK"]
    fold = np.repeat(g["dKslc"], S, axis=1) / S
    assert np.allclose(diff[:, :nC * S], fold, rtol=1e-12, atol=1e-14)
    assert np.all(g["dK"][:, nC * S:] == 0) and np.all(g["dV"][:, nC * S:] == 0)


def pin_backward_masks(orc):
    """Masked backward (only some tokens' dQ and some chunks' dK/dV asked for) returns the
    same values as the full backward where asked."""
    gen = torch.Generator().manual_seed(14)
    B, S, Hq, Hkv, D, K = 2, 8, 4, 2, 8, 3
    L = 9 * S
    Q, Km, V, dO = (_rand(gen, (B, L, h, D), 1.0, torch.float32) for h in (Hq, Hkv, Hkv, Hq))
    Qs = _rand(gen, (B, L, Hkv, D), 1.0, torch.float32)
    f = orc.forward(Q, Km, V, Qs, S, K)
    full = orc.backward(Q, Km, V, Qs, f["Kslc"], f["idx"], f["score"], f["w"], dO, S)
    tm = np.zeros((B, L), np.uint8)
    tm[0, 40] = tm[1, 70] = 1
    cm = np.zeros((B, L // S), np.uint8)
    cm[0, 1] = cm[1, 4] = 1
    part = orc.backward(Q, Km, V, Qs, f["Kslc"], f["idx"], f["score"], f["w"], dO, S,
                        tok_mask=tm, chunk_mask=cm)
    for (b, t) in ((0, 40), (1, 70)):
        assert np.array_equal(part["dQ"][b, t], full["dQ"][b, t])
        assert np.array_equal(part["dQs"][b, t], full["dQs"][b, t])
    for (b, c) in ((0, 1), (1, 4)):
        sl = slice(c * S, (c + 1) * S)
        assert np.array_equal(part["dK"][b, sl], full["dK"][b, sl])
        assert np.array_equal(part["dV"][b, sl], full["dV"][b, sl])
        assert np.array_equal(part["dKslc"][b, c], full["dKslc"][b, c])


# ----------------------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------------------
def pin_decode_equals_forward_row(orc):
    """A decode step at context length t returns what the forward returns for token t."""
    gen = torch.Generator().manual_seed(15)
    S, Hq, Hkv, D, K = 8, 4, 2, 8, 3
    L = 12 * S
    Q = _rand(gen, (1, L, Hq, D), 0.5, torch.bfloat16)
    Km = _rand(gen, (1, L, Hkv, D), 0.5, torch.bfloat16)
    V = _rand(gen, (1, L, Hkv, D), 0.5, torch.bfloat16)
    Qs = _rand(gen, (1, L, Hkv, D), 1.0, torch.bfloat16)
    for weights in ("stick", "softmax"):
        f = orc.forward(Q, Km, V, Qs, S, K, weights=weights)
        for t in (S - 1, S, 3 * S + 2, 7 * S, L - 1):
            ctx = t
            ks = orc.pool(Km[:, :ctx], S)
            d = orc.decode(Q[:, t], Qs[:, t], Km[:, :ctx], V[:, :ctx], ks, S, K, weights=weights)
            assert np.array_equal(d["idx"], f["idx"][:, t]), t
            assert np.allclose(d["w"], f["w"][:, t], rtol=0, atol=0), t
            assert np.allclose(d["O"], f["O"][:, t], rtol=1e-13, atol=1e-14), t


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
