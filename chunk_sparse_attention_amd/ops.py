"""Tensor-level Python binding of libhsa.so: argument marshalling only.

Each function checks that its tensors are contiguous device tensors of the expected dtype,
allocates the outputs (and the workspace, unless one is passed), and calls the C entry
point of the same name on torch's current stream.  Every step of the computation runs in
the library's HIP kernels.

Shapes (BSHD, see include/hsa.h):
    Q, dO, O  [B, L, Hq, D]       K, V, Qs  [B, L, Hkv, D]      Kslc [B, L//64, Hkv, D]
    idx [B, L, Hkv, K] int32      score, w  [B, L, Hkv, K] fp32
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import Problem, check

S_CHUNK = 64
_DT = {torch.float32: _lib.HSA_F32, torch.bfloat16: _lib.HSA_BF16}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the operator has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def problem(B, L, Hq, Hkv, D, K, dtype, sm_scale=None, sel_scale=None, generic=False,
            S=S_CHUNK, weights="stick") -> Problem:
    """weights: "stick" (stick-breaking chunk weights) or "softmax" (a softmax of the
    selected chunks' scores, HSA_FLAG_SOFTMAX_WEIGHTS)."""
    if dtype not in _DT:
        raise TypeError(f"unsupported dtype {dtype}")
    if weights not in ("stick", "softmax"):
        raise ValueError(f"weights must be 'stick' or 'softmax', not {weights!r}")
    flags = (_lib.HSA_FLAG_GENERIC if generic else 0) | (
        _lib.HSA_FLAG_SOFTMAX_WEIGHTS if weights == "softmax" else 0)
    return Problem(int(B), int(L), int(Hq), int(Hkv), int(D), int(S), int(K),
                   0.0 if sm_scale is None else float(sm_scale),
                   0.0 if sel_scale is None else float(sel_scale), _DT[dtype], flags)


def workspace_size(op: int, prob: Problem) -> int:
    n = ctypes.c_size_t(0)
    check(_lib.lib().hsa_workspace_size(int(op), ctypes.byref(prob), ctypes.byref(n)),
          "hsa_workspace_size")
    return int(n.value)


def workspace(op: int, prob: Problem, device) -> torch.Tensor | None:
    n = workspace_size(op, prob)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _ws_args(ws):
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


def pool(K: torch.Tensor, K_top: int = 1, generic=False) -> torch.Tensor:
    """Chunk keys Kslc = mean of each chunk's key rows (hsa_select with Qs = NULL)."""
    _need(K, "K")
    B, L, Hkv, D = K.shape
    prob = problem(B, L, Hkv, Hkv, D, K_top, K.dtype, generic=generic)
    Kslc = torch.empty((B, L // S_CHUNK, Hkv, D), dtype=K.dtype, device=K.device)
    ws = workspace(_lib.HSA_OP_SELECT, prob, K.device)
    wp, wn = _ws_args(ws)
    check(_lib.lib().hsa_select(ctypes.byref(prob), None, _ptr(K), _ptr(Kslc), None, None, None,
                                wp, wn, _stream()), "hsa_select")
    return Kslc


def select(Qs: torch.Tensor, K: torch.Tensor, K_top: int, sel_scale=None, generic=False,
           ws=None, weights="stick"):
    """Pool + top-K selection + chunk weights (stick-breaking, or softmax with
    weights="softmax").  Returns (Kslc, idx, score, w)."""
    _need(K, "K")
    B, L, Hkv, D = K.shape
    _need(Qs, "Qs", K.dtype, (B, L, Hkv, D), K.device)
    prob = problem(B, L, Hkv, Hkv, D, K_top, K.dtype, sel_scale=sel_scale, generic=generic,
                   weights=weights)
    dev = K.device
    Kslc = torch.empty((B, L // S_CHUNK, Hkv, D), dtype=K.dtype, device=dev)
    idx = torch.empty((B, L, Hkv, K_top), dtype=torch.int32, device=dev)
    score = torch.empty((B, L, Hkv, K_top), dtype=torch.float32, device=dev)
    w = torch.empty((B, L, Hkv, K_top), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(_lib.HSA_OP_SELECT, prob, dev)
    wp, wn = _ws_args(ws)
    check(_lib.lib().hsa_select(ctypes.byref(prob), _ptr(Qs), _ptr(K), _ptr(Kslc), _ptr(idx),
                                _ptr(score), _ptr(w), wp, wn, _stream()), "hsa_select")
    return Kslc, idx, score, w


def fwd(Q, K, V, idx, w, sm_scale=None, generic=False, ws=None, out=None, want_lse=False):
    """O = sum_k w_k softmax1-attention of Q over the selected chunks of K/V.
    want_lse=True returns (O, lse) with lse [B, L, Hq, K] fp32: every (token, head, slot)'s
    softmax-off-by-one normaliser log(1 + sum_j exp(z_j)), 0 for masked slots."""
    _need(Q, "Q")
    B, L, Hq, D = Q.shape
    Hkv = K.shape[2]
    Kt = idx.shape[-1]
    _need(K, "K", Q.dtype, (B, L, Hkv, D), Q.device)
    _need(V, "V", Q.dtype, (B, L, Hkv, D), Q.device)
    _need(idx, "idx", torch.int32, (B, L, Hkv, Kt), Q.device)
    _need(w, "w", torch.float32, (B, L, Hkv, Kt), Q.device)
    prob = problem(B, L, Hq, Hkv, D, Kt, Q.dtype, sm_scale=sm_scale, generic=generic)
    O = torch.empty_like(Q) if out is None else _need(out, "out", Q.dtype, Q.shape, Q.device)
    lse = (torch.empty((B, L, Hq, Kt), dtype=torch.float32, device=Q.device)
           if want_lse else None)
    if ws is None:
        ws = workspace(_lib.HSA_OP_FWD, prob, Q.device)
    wp, wn = _ws_args(ws)
    check(_lib.lib().hsa_fwd(ctypes.byref(prob), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx), _ptr(w),
                             _ptr(O), _ptr(lse), wp, wn, _stream()), "hsa_fwd")
    return (O, lse) if want_lse else O


def bwd(Q, K, V, Qs, Kslc, idx, score, w, dO, fold=True, want_dkslc=True, sm_scale=None,
        sel_scale=None, generic=False, ws=None, after_fwd=False, weights="stick", lse=None):
    """Gradients with the selection fixed.  Returns dict(dQ, dK, dV, dQs, dKslc).
    weights: the chunk-weight rule select() used ("stick" or "softmax").
    lse: the normalisers fwd(want_lse=True) returned for the same Q, K and idx (optional).

    after_fwd=True: `ws` is the workspace that fwd() just used for the same Q, K, idx and w
    (allocate it with workspace(HSA_OP_BWD, ...), which also fits the forward); the backward
    then reuses the state the forward left in it (HSA_BWD_AFTER_FWD) when the library's
    record of that workspace confirms it, and rebuilds it otherwise."""
    _need(Q, "Q")
    B, L, Hq, D = Q.shape
    Hkv = K.shape[2]
    Kt = idx.shape[-1]
    dev = Q.device
    for name, t, h in (("K", K, Hkv), ("V", V, Hkv), ("Qs", Qs, Hkv), ("dO", dO, Hq)):
        _need(t, name, Q.dtype, (B, L, h, D), dev)
    _need(Kslc, "Kslc", Q.dtype, (B, L // S_CHUNK, Hkv, D), dev)
    _need(idx, "idx", torch.int32, (B, L, Hkv, Kt), dev)
    _need(score, "score", torch.float32, (B, L, Hkv, Kt), dev)
    _need(w, "w", torch.float32, (B, L, Hkv, Kt), dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, L, Hq, Kt), dev)
    prob = problem(B, L, Hq, Hkv, D, Kt, Q.dtype, sm_scale=sm_scale, sel_scale=sel_scale,
                   generic=generic, weights=weights)
    dQ = torch.empty_like(Q)
    dK = torch.empty_like(K)
    dV = torch.empty_like(V)
    dQs = torch.empty_like(Qs)
    dKslc = (torch.empty((B, L // S_CHUNK, Hkv, D), dtype=torch.float32, device=dev)
             if want_dkslc else None)
    if ws is None:
        if after_fwd:
            raise ValueError("after_fwd needs the workspace the forward used")
        ws = workspace(_lib.HSA_OP_BWD, prob, dev)
    wp, wn = _ws_args(ws)
    flags = (_lib.HSA_BWD_FOLD_KSLC if fold else 0) | (_lib.HSA_BWD_AFTER_FWD if after_fwd else 0)
    check(_lib.lib().hsa_bwd(ctypes.byref(prob), _ptr(Q), _ptr(K), _ptr(V), _ptr(Qs), _ptr(Kslc),
                             _ptr(idx), _ptr(score), _ptr(w), _ptr(lse), _ptr(dO), _ptr(dQ),
                             _ptr(dK), _ptr(dV), _ptr(dQs), _ptr(dKslc), flags, wp, wn,
                             _stream()),
          "hsa_bwd")
    return dict(dQ=dQ, dK=dK, dV=dV, dQs=dQs, dKslc=dKslc)


def decode(q, qs, Kc, Vc, Kslc, K_top, sm_scale=None, sel_scale=None, generic=False, ws=None,
           weights="stick"):
    """One decode step: q [B,Hq,D], qs [B,Hkv,D], caches [B,ctx,Hkv,D], Kslc [B,ctx//64,Hkv,D].
    Returns (O [B,Hq,D], idx, score, w [B,Hkv,K])."""
    _need(Kc, "Kcache")
    B, ctx, Hkv, D = Kc.shape
    dev = Kc.device
    Hq = q.shape[1]
    _need(q, "q", Kc.dtype, (B, Hq, D), dev)
    _need(qs, "qs", Kc.dtype, (B, Hkv, D), dev)
    _need(Vc, "Vcache", Kc.dtype, (B, ctx, Hkv, D), dev)
    _need(Kslc, "Kslc", Kc.dtype, (B, ctx // S_CHUNK, Hkv, D), dev)
    prob = problem(B, ctx, Hq, Hkv, D, K_top, Kc.dtype, sm_scale=sm_scale, sel_scale=sel_scale,
                   generic=generic, weights=weights)
    O = torch.empty((B, Hq, D), dtype=Kc.dtype, device=dev)
    idx = torch.empty((B, Hkv, K_top), dtype=torch.int32, device=dev)
    score = torch.empty((B, Hkv, K_top), dtype=torch.float32, device=dev)
    w = torch.empty((B, Hkv, K_top), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(_lib.HSA_OP_DECODE, prob, dev)
    wp, wn = _ws_args(ws)
    check(_lib.lib().hsa_decode(ctypes.byref(prob), _ptr(q), _ptr(qs), _ptr(Kc), _ptr(Vc),
                                _ptr(Kslc), _ptr(O), _ptr(idx), _ptr(score), _ptr(w), wp, wn,
                                _stream()), "hsa_decode")
    return O, idx, score, w


def decode_host_kv(q, qs, Kc, Vc, Kslc, K_top, sm_scale=None, sel_scale=None, generic=False,
                   ws=None, weights="stick"):
    """decode() with the caches Kc, Vc [B,ctx,Hkv,D] in pinned host memory (CPU tensors made
    with pin_memory); the step reads only the selected chunks' rows of them.  q, qs and Kslc
    are GPU tensors.  Returns (O [B,Hq,D], idx, score, w [B,Hkv,K])."""
    for t, name in ((Kc, "Kcache"), (Vc, "Vcache")):
        if not isinstance(t, torch.Tensor) or t.is_cuda or not t.is_pinned():
            raise ValueError(f"{name} must be a pinned host tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, ctx, Hkv, D = Kc.shape
    if Vc.dtype != Kc.dtype or tuple(Vc.shape) != tuple(Kc.shape):
        raise ValueError("Vcache must match Kcache in dtype and shape")
    _need(q, "q", Kc.dtype)
    dev = q.device
    Hq = q.shape[1]
    _need(q, "q", Kc.dtype, (B, Hq, D), dev)
    _need(qs, "qs", Kc.dtype, (B, Hkv, D), dev)
    _need(Kslc, "Kslc", Kc.dtype, (B, ctx // S_CHUNK, Hkv, D), dev)
    prob = problem(B, ctx, Hq, Hkv, D, K_top, Kc.dtype, sm_scale=sm_scale, sel_scale=sel_scale,
                   generic=generic, weights=weights)
    O = torch.empty((B, Hq, D), dtype=Kc.dtype, device=dev)
    idx = torch.empty((B, Hkv, K_top), dtype=torch.int32, device=dev)
    score = torch.empty((B, Hkv, K_top), dtype=torch.float32, device=dev)
    w = torch.empty((B, Hkv, K_top), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(_lib.HSA_OP_DECODE, prob, dev)
    wp, wn = _ws_args(ws)
    check(_lib.lib().hsa_decode_host_kv(ctypes.byref(prob), _ptr(q), _ptr(qs), _ptr(Kc),
                                        _ptr(Vc), _ptr(Kslc), _ptr(O), _ptr(idx), _ptr(score),
                                        _ptr(w), wp, wn, _stream()), "hsa_decode_host_kv")
    return O, idx, score, w


def decode_ragged(q, qs, Kc, Vc, Kslc, ctx_lens, K_top, sm_scale=None, sel_scale=None,
                  generic=False, ws=None, weights="stick"):
    """decode() for sequences of different lengths in one cache: ctx_lens [B] int32 (GPU),
    caches [B,L,Hkv,D] with L the capacity.  Returns (O [B,Hq,D], idx, score, w [B,Hkv,K])."""
    _need(Kc, "Kcache")
    B, ctx, Hkv, D = Kc.shape
    dev = Kc.device
    Hq = q.shape[1]
    _need(q, "q", Kc.dtype, (B, Hq, D), dev)
    _need(qs, "qs", Kc.dtype, (B, Hkv, D), dev)
    _need(Vc, "Vcache", Kc.dtype, (B, ctx, Hkv, D), dev)
    _need(Kslc, "Kslc", Kc.dtype, (B, ctx // S_CHUNK, Hkv, D), dev)
    _need(ctx_lens, "ctx_lens", torch.int32, (B,), dev)
    prob = problem(B, ctx, Hq, Hkv, D, K_top, Kc.dtype, sm_scale=sm_scale, sel_scale=sel_scale,
                   generic=generic, weights=weights)
    O = torch.empty((B, Hq, D), dtype=Kc.dtype, device=dev)
    idx = torch.empty((B, Hkv, K_top), dtype=torch.int32, device=dev)
    score = torch.empty((B, Hkv, K_top), dtype=torch.float32, device=dev)
    w = torch.empty((B, Hkv, K_top), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(_lib.HSA_OP_DECODE, prob, dev)
    wp, wn = _ws_args(ws)
    check(_lib.lib().hsa_decode_ragged(ctypes.byref(prob), _ptr(ctx_lens), _ptr(q), _ptr(qs),
                                       _ptr(Kc), _ptr(Vc), _ptr(Kslc), _ptr(O), _ptr(idx),
                                       _ptr(score), _ptr(w), wp, wn, _stream()),
          "hsa_decode_ragged")
    return O, idx, score, w


def pool_chunks(K, Kslc, chunk_ids):
    """Recompute Kslc[b, c] in place for the chunks c listed in chunk_ids [B, n] int32 (GPU;
    entries outside [0, nC) are skipped).  K [B,L,Hkv,D], Kslc [B,L//64,Hkv,D]."""
    _need(K, "K")
    B, L, Hkv, D = K.shape
    _need(Kslc, "Kslc", K.dtype, (B, L // S_CHUNK, Hkv, D), K.device)
    _need(chunk_ids, "chunk_ids", torch.int32, None, K.device)
    if chunk_ids.dim() != 2 or chunk_ids.shape[0] != B:
        raise ValueError(f"chunk_ids must be [B={B}, n], not {tuple(chunk_ids.shape)}")
    prob = problem(B, L, Hkv, Hkv, D, 1, K.dtype)
    check(_lib.lib().hsa_pool_chunks(ctypes.byref(prob), _ptr(K), _ptr(Kslc), _ptr(chunk_ids),
                                     int(chunk_ids.shape[1]), _stream()), "hsa_pool_chunks")
    return Kslc


def fwd_layers(Q, K, V, idx, w, sm_scale=None, generic=False, ws=None, out=None):
    """fwd() for a stack of layers sharing one selection: Q [n,B,L,Hq,D], K, V [n,B,L,Hkv,D],
    idx/w [B,L,Hkv,K].  Returns O [n,B,L,Hq,D]."""
    _need(Q, "Q")
    n, B, L, Hq, D = Q.shape
    Hkv = K.shape[3]
    Kt = idx.shape[-1]
    _need(K, "K", Q.dtype, (n, B, L, Hkv, D), Q.device)
    _need(V, "V", Q.dtype, (n, B, L, Hkv, D), Q.device)
    _need(idx, "idx", torch.int32, (B, L, Hkv, Kt), Q.device)
    _need(w, "w", torch.float32, (B, L, Hkv, Kt), Q.device)
    prob = problem(B, L, Hq, Hkv, D, Kt, Q.dtype, sm_scale=sm_scale, generic=generic)
    O = torch.empty_like(Q) if out is None else _need(out, "out", Q.dtype, Q.shape, Q.device)
    if ws is None:
        ws = workspace(_lib.HSA_OP_FWD, prob, Q.device)
    wp, wn = _ws_args(ws)
    check(_lib.lib().hsa_fwd_layers(ctypes.byref(prob), n, _ptr(Q), _ptr(K), _ptr(V),
                                    _ptr(idx), _ptr(w), _ptr(O), wp, wn, _stream()),
          "hsa_fwd_layers")
    return O


def decode_shared(q, Kc, Vc, idx, w, sm_scale=None):
    """Decode attention of a stack of layers with a selection made before (idx/w [B,Hkv,K]
    from decode()): q [n,B,Hq,D], caches [n,B,ctx,Hkv,D] on the GPU, or pinned host tensors
    (the host-cache variant).  Returns O [n,B,Hq,D]."""
    host = not Kc.is_cuda
    if host:
        for t, name in ((Kc, "Kcache"), (Vc, "Vcache")):
            if not isinstance(t, torch.Tensor) or t.is_cuda or not t.is_pinned():
                raise ValueError(f"{name} must be a GPU tensor or a pinned host tensor")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
    else:
        _need(Kc, "Kcache")
    n, B, ctx, Hkv, D = Kc.shape
    dev = q.device
    Hq = q.shape[2]
    K_top = idx.shape[-1]
    _need(q, "q", Kc.dtype, (n, B, Hq, D), dev)
    if host:
        if Vc.dtype != Kc.dtype or tuple(Vc.shape) != tuple(Kc.shape):
            raise ValueError("Vcache must match Kcache in dtype and shape")
    else:
        _need(Vc, "Vcache", Kc.dtype, (n, B, ctx, Hkv, D), dev)
    _need(idx, "idx", torch.int32, (B, Hkv, K_top), dev)
    _need(w, "w", torch.float32, (B, Hkv, K_top), dev)
    prob = problem(B, ctx, Hq, Hkv, D, K_top, Kc.dtype, sm_scale=sm_scale)
    O = torch.empty((n, B, Hq, D), dtype=Kc.dtype, device=dev)
    fn = _lib.lib().hsa_decode_shared_host_kv if host else _lib.lib().hsa_decode_shared
    check(fn(ctypes.byref(prob), n, _ptr(q), _ptr(Kc), _ptr(Vc), _ptr(idx), _ptr(w), _ptr(O),
             _stream()), "hsa_decode_shared_host_kv" if host else "hsa_decode_shared")
    return O


def timer_enable(on: bool = True) -> None:
    """Start (forgetting earlier records) or stop HIP-event timing of every kernel launch."""
    check(_lib.lib().hsa_timer_enable(1 if on else 0), "hsa_timer_enable")


def timer_read() -> dict:
    """{kernel class: (recorded launches, total ms)} since the last timer_enable(True)."""
    out = {}
    for i, name in enumerate(_lib.KERNEL_CLASSES):
        n, ms = ctypes.c_int(0), ctypes.c_double(0.0)
        check(_lib.lib().hsa_timer_read(i, ctypes.byref(n), ctypes.byref(ms)), "hsa_timer_read")
        out[name] = (int(n.value), float(ms.value))
    return out
