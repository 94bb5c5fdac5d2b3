"""Seeded synthetic inputs for the HSA operator.

This module serves both the GPU library's tests/benchmark and the CPU oracle's tests.  It
holds only random-number recipes and shapes -- none of the method's arithmetic (no pooling,
scoring, ranking, weighting or attention).

Workloads (the pages' regime: contexts of 16K tokens and more, chunk size S = 64):

  tiny_fp32    B=1  L=1024    Hq=4  Hkv=1 d=64  K=4  fp32   Q,K,V,Qs ~ N(0,1)
  fwd_16k      B=4  L=16384   Hq=16 Hkv=2 d=64  K=8  bf16   Q,K,V ~ 0.5 N(0,1), Qs ~ N(0,1)
  fwd_64k      B=1  L=65536   Hq=16 Hkv=2 d=128 K=8  bf16   as fwd_16k, plus a planted
               direction u: 1% of chunks get +2u on every key row, and a random 5% of
               tokens get +2u on their selection query (both groups)
  bwd_16k      B=2  L=16384   Hq=16 Hkv=2 d=64  K=8  bf16   as fwd_16k, dO ~ N(0,1)
  decode_1m    B=16 ctx=2^20  Hq=16 Hkv=2 d=64  K=8  bf16   K,V ~ 0.5 N(0,1); q ~ 0.5 N(0,1),
               qs ~ N(0,1); one new token per sequence

Recipe: one CPU ``torch.Generator`` seeded with ``seed``; draws in the order Q, K, V, Qs,
dO (then u, the chunk permutation and the token permutation for fwd_64k); every draw is
fp32 N(0,1), scaled, shifted in fp32 and only then rounded to the storage type.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    L: int
    Hq: int
    Hkv: int
    D: int
    S: int
    K: int
    dtype: torch.dtype
    qkv_std: float = 0.5
    qs_std: float = 1.0
    planted: bool = False  # the fwd_64k planted-direction structure
    decode: bool = False

    @property
    def nC(self) -> int:
        return self.L // self.S

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 1024, 4, 1, 64, 64, 4, torch.float32, 1.0, 1.0),
    "fwd_16k": Workload("fwd_16k", 4, 16384, 16, 2, 64, 64, 8, torch.bfloat16),
    "fwd_64k": Workload("fwd_64k", 1, 65536, 16, 2, 128, 64, 8, torch.bfloat16, planted=True),
    "bwd_16k": Workload("bwd_16k", 2, 16384, 16, 2, 64, 64, 8, torch.bfloat16),
    "decode_1m": Workload("decode_1m", 16, 1 << 20, 16, 2, 64, 64, 8, torch.bfloat16,
                          decode=True),
}


def _randn(gen, shape, std):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def make_inputs(wl: Workload, seed: int = 0, with_grad: bool = True) -> dict:
    """Host tensors Q [B,L,Hq,D], K, V, Qs [B,L,Hkv,D] and dO [B,L,Hq,D] in wl.dtype."""
    assert not wl.decode
    gen = torch.Generator().manual_seed(seed)
    B, L, Hq, Hkv, D = wl.B, wl.L, wl.Hq, wl.Hkv, wl.D
    Q = _randn(gen, (B, L, Hq, D), wl.qkv_std)
    K = _randn(gen, (B, L, Hkv, D), wl.qkv_std)
    V = _randn(gen, (B, L, Hkv, D), wl.qkv_std)
    Qs = _randn(gen, (B, L, Hkv, D), wl.qs_std)
    dO = _randn(gen, (B, L, Hq, D), 1.0) if with_grad else None
    meta = {}
    if wl.planted:
        n = torch.randn((D,), generator=gen, dtype=torch.float32)
        u = n / n.norm()
        n_chunks = int(round(0.01 * wl.nC))
        n_tokens = int(round(0.05 * L))
        chunks = torch.randperm(wl.nC, generator=gen)[:n_chunks]
        tokens = torch.randperm(L, generator=gen)[:n_tokens]
        for c in chunks.tolist():
            K[:, c * wl.S:(c + 1) * wl.S, :, :] += 2.0 * u
        Qs[:, tokens, :, :] += 2.0 * u
        meta = dict(u=u, planted_chunks=chunks, planted_tokens=tokens)
    out = dict(Q=Q.to(wl.dtype), K=K.to(wl.dtype), V=V.to(wl.dtype), Qs=Qs.to(wl.dtype))
    if dO is not None:
        out["dO"] = dO.to(wl.dtype)
    out.update(meta)
    return out


def make_decode_inputs(wl: Workload, seed: int = 0, ctx: int | None = None,
                       slab: int = 1) -> dict:
    """Host tensors for one decode step: q [B,Hq,D], qs [B,Hkv,D], Kc/Vc [B,ctx,Hkv,D].
    The caches are drawn ``slab`` sequences at a time to bound the fp32 staging memory."""
    gen = torch.Generator().manual_seed(seed)
    B, Hq, Hkv, D = wl.B, wl.Hq, wl.Hkv, wl.D
    ctx = wl.L if ctx is None else ctx
    q = _randn(gen, (B, Hq, D), wl.qkv_std).to(wl.dtype)
    qs = _randn(gen, (B, Hkv, D), wl.qs_std).to(wl.dtype)
    Kc = torch.empty((B, ctx, Hkv, D), dtype=wl.dtype)
    Vc = torch.empty((B, ctx, Hkv, D), dtype=wl.dtype)
    for dst in (Kc, Vc):
        for b0 in range(0, B, slab):
            b1 = min(B, b0 + slab)
            dst[b0:b1] = _randn(gen, (b1 - b0, ctx, Hkv, D), wl.qkv_std).to(wl.dtype)
    return dict(q=q, qs=qs, Kc=Kc, Vc=Vc)


def make_selection(B: int, L: int, Hkv: int, S: int, K: int, seed: int = 0,
                   nC: int | None = None) -> dict:
    """A random valid causal selection, given to both sides when the attention and backward
    steps are tested apart from selection: for each (b, t, g) a random set of
    min(K, floor(t/S)) distinct earlier chunks in random order, random scores sorted
    descending (fp32), random positive weights (fp32), masked slots idx -1 / -inf / 0."""
    gen = torch.Generator().manual_seed(seed)
    nC = L // S if nC is None else nC
    idx = torch.full((B, L, Hkv, K), -1, dtype=torch.int32)
    score = torch.full((B, L, Hkv, K), float("-inf"), dtype=torch.float32)
    w = torch.zeros((B, L, Hkv, K), dtype=torch.float32)
    # one random key per (row, chunk); the K smallest among the available chunks are taken
    for qc in range(1, nC + 1):
        t0, t1 = qc * S, min(L, (qc + 1) * S)
        if t0 >= L:
            break
        n_av = min(qc, nC)
        nv = min(K, n_av)
        keys = torch.rand((B, t1 - t0, Hkv, n_av), generator=gen)
        chosen = keys.argsort(dim=-1)[..., :nv].to(torch.int32)
        idx[:, t0:t1, :, :nv] = chosen
        sc = torch.randn((B, t1 - t0, Hkv, nv), generator=gen).sort(dim=-1, descending=True)
        score[:, t0:t1, :, :nv] = sc.values
        w[:, t0:t1, :, :nv] = torch.rand((B, t1 - t0, Hkv, nv), generator=gen) * 0.3 + 0.01
    return dict(idx=idx, score=score, w=w)

