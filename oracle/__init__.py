"""CPU oracle for Hierarchical Sparse Attention (HSA) -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The GPU library never links, loads or calls it, and this
package never imports the GPU library: the two share no code.

The arithmetic lives in ``hsa_oracle.c`` (plain C, IEEE double, one loop per step of the
method).  This module only builds that file with gcc, marshals numpy / torch-CPU arrays
into it, and returns float64 numpy arrays.

Sources: "Hardware-aligned Hierarchical Sparse Attention for Efficient Long-term Memory
Access" -- papernotes.org note, section 方法详解 (层次化稀疏注意力（HSA）, 硬件对齐 Kernel,
训练与推理优化); atlas.scime.ai summary, section "Approach".  The step-by-step citations
are in the C file next to each function.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import tempfile

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, F64 = 0, 1, 2


def build(out: str = _LIB, mutation: int = 0) -> str:
    """Compile the oracle with gcc (no fast-math).  ``mutation`` != 0 builds a copy with one
    planted mistake; it is used only by the oracle's self-tests."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-Wall",
           f"-DORACLE_MUTATION={int(mutation)}", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_mutant(mutation: int) -> "Oracle":
    d = tempfile.mkdtemp(prefix="hsa_oracle_mut")
    path = build(os.path.join(d, f"liboracle_m{mutation}.so"), mutation)
    return Oracle(path)


_P = ctypes.c_void_p
_I = ctypes.c_int
_D = ctypes.c_double


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as_storage(x):
    """Return (contiguous numpy array in its storage type, dtype code)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            if x.dtype == torch.float64:
                return x.numpy(), F64
            raise TypeError(f"unsupported tensor dtype {x.dtype}")
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, BF16
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.float64:
        return x, F64
    raise TypeError(f"unsupported array dtype {x.dtype}")


def _f64(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().double().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x, dtype=np.float64)


def _i32(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x, dtype=np.int32)


def _wmode(weights: str) -> int:
    """Chunk-weight mode of the C oracle: 0 stick-breaking, 1 softmax."""
    modes = {"stick": 0, "softmax": 1}
    if weights not in modes:
        raise ValueError(f"weights must be one of {sorted(modes)}")
    return modes[weights]


def _mask(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x).reshape(-1), dtype=np.uint8)


class Oracle:
    """ctypes handle on one build of hsa_oracle.c."""

    def __init__(self, path: str = _LIB):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_set_threads.restype = None
        lib.oracle_set_threads.argtypes = [_I]
        lib.oracle_max_threads.restype = _I
        lib.oracle_max_threads.argtypes = []
        lib.oracle_round.restype = _D
        lib.oracle_round.argtypes = [_D, _I]
        lib.oracle_pool.restype = None
        lib.oracle_pool.argtypes = [_P, _I, _I, _I, _I, _I, _I, _I, _P]
        lib.oracle_select.restype = None
        lib.oracle_select.argtypes = [_P, _I, _P, _I, _I, _I, _I, _I, _I, _D, _I, _I, _P, _P, _P,
                                      _P]
        lib.oracle_attend.restype = None
        lib.oracle_attend.argtypes = [_P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _I, _D,
                                      _P, _P, _P, _P]
        lib.oracle_bwd.restype = None
        lib.oracle_bwd.argtypes = [_P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                   _I, _I, _D, _D, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        lib.oracle_decode.restype = None
        lib.oracle_decode.argtypes = [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _D, _D,
                                      _I, _I, _P, _P, _P, _P]
        self.lib = lib

    # -- threads -------------------------------------------------------------------------
    def set_threads(self, n: int) -> None:
        """OpenMP threads of the row loops from now on (results do not depend on it)."""
        self.lib.oracle_set_threads(int(n))

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    # -- elementwise -------------------------------------------------------------------
    def round(self, x: float, dt: int) -> float:
        """Round to the nearest value of storage type ``dt`` (F32 or BF16), ties to even."""
        return self.lib.oracle_round(float(x), int(dt))

    # -- F1 ------------------------------------------------------------------------------
    def pool(self, K, S: int, round_dt: int | None = None):
        """Chunk keys Kslc[b,c,g,:] = mean_j K[b,cS+j,g,:], rounded once to ``round_dt``
        (default: the storage type of K).  Returns float64 [B, L//S, Hkv, D]."""
        k, dt = _as_storage(K)
        B, L, Hkv, D = k.shape
        nC = L // S
        out = np.zeros((B, nC, Hkv, D), np.float64)
        self.lib.oracle_pool(_ptr(k), dt, B, L, Hkv, D, S, dt if round_dt is None else round_dt,
                             _ptr(out))
        return out

    # -- F2-F4 ---------------------------------------------------------------------------
    def select(self, Qs, Kslc, S: int, K: int, sel_scale: float | None = None,
               score_dt: int = F32, row_mask=None, weights: str = "stick"):
        """Top-K chunk selection + chunk weights (weights="stick": stick-breaking, "softmax":
        softmax of the valid slots' scores).  Returns (idx int32, score f64, w f64), each
        [B, L, Hkv, K]."""
        qs, dt = _as_storage(Qs)
        B, L, Hkv, D = qs.shape
        ks = _f64(Kslc)
        assert ks.shape == (B, L // S, Hkv, D), ks.shape
        if sel_scale is None:
            sel_scale = 1.0 / math.sqrt(D)
        idx = np.full((B, L, Hkv, K), -1, np.int32)
        score = np.full((B, L, Hkv, K), -np.inf, np.float64)
        w = np.zeros((B, L, Hkv, K), np.float64)
        m = _mask(row_mask)
        self.lib.oracle_select(_ptr(qs), dt, _ptr(ks), B, L, Hkv, D, S, K, float(sel_scale),
                               score_dt, _wmode(weights), _ptr(m), _ptr(idx), _ptr(score),
                               _ptr(w))
        return idx, score, w

    # -- F5-F6 ---------------------------------------------------------------------------
    def attend(self, Q, Kmat, V, idx, w, S: int, sm_scale: float | None = None,
               row_mask=None, per_slot: bool = False, want_lse: bool = False):
        """O = sum_k w_k softmax1-attention over the selected chunks.
        Returns O float64 [B, L, Hq, D], followed, when asked, by the per-slot outputs
        [B, L, Hq, K, D] and by lse [B, L, Hq, K] = log(1 + sum_j exp(z_j)) of every
        (token, head, slot) (0 for masked slots)."""
        q, dt = _as_storage(Q)
        k, dtk = _as_storage(Kmat)
        v, dtv = _as_storage(V)
        assert dt == dtk == dtv
        B, L, Hq, D = q.shape
        Hkv = k.shape[2]
        idx_ = _i32(idx)
        w_ = _f64(w)
        Kt = idx_.shape[-1]
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(D)
        O = np.zeros((B, L, Hq, D), np.float64)
        Ok = np.zeros((B, L, Hq, Kt, D), np.float64) if per_slot else None
        lse = np.zeros((B, L, Hq, Kt), np.float64) if want_lse else None
        m = _mask(row_mask)
        self.lib.oracle_attend(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(idx_), _ptr(w_), B, L, Hq,
                               Hkv, D, S, Kt, float(sm_scale), _ptr(m), _ptr(O), _ptr(Ok),
                               _ptr(lse))
        out = (O,) + ((Ok,) if per_slot else ()) + ((lse,) if want_lse else ())
        return out if len(out) > 1 else O

    def forward(self, Q, Kmat, V, Qs, S: int, K: int, sm_scale=None, sel_scale=None,
                score_dt: int = F32, row_mask=None, weights: str = "stick"):
        """pool -> select -> attend.  Returns dict(Kslc, idx, score, w, O)."""
        Kslc = self.pool(Kmat, S)
        idx, score, w = self.select(Qs, Kslc, S, K, sel_scale, score_dt, row_mask, weights)
        O = self.attend(Q, Kmat, V, idx, w, S, sm_scale, row_mask)
        return dict(Kslc=Kslc, idx=idx, score=score, w=w, O=O)

    # -- B1-B5 ---------------------------------------------------------------------------
    def backward(self, Q, Kmat, V, Qs, Kslc, idx, score, w, dO, S: int, sm_scale=None,
                 sel_scale=None, fold: bool = True, tok_mask=None, chunk_mask=None,
                 weights: str = "stick"):
        """Gradients with the selection held fixed.  Returns dict(dQ, dK, dV, dQs, dKslc, dw,
        ds) as float64 arrays."""
        q, dt = _as_storage(Q)
        k, _ = _as_storage(Kmat)
        v, _ = _as_storage(V)
        qs, _ = _as_storage(Qs)
        do, _ = _as_storage(dO)
        B, L, Hq, D = q.shape
        Hkv = k.shape[2]
        nC = L // S
        idx_ = _i32(idx)
        Kt = idx_.shape[-1]
        sc = _f64(score)
        w_ = _f64(w)
        ks = _f64(Kslc)
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(D)
        if sel_scale is None:
            sel_scale = 1.0 / math.sqrt(D)
        out = dict(
            dQ=np.zeros((B, L, Hq, D)), dK=np.zeros((B, L, Hkv, D)), dV=np.zeros((B, L, Hkv, D)),
            dQs=np.zeros((B, L, Hkv, D)), dKslc=np.zeros((B, nC, Hkv, D)),
            dw=np.zeros((B, L, Hkv, Kt)), ds=np.zeros((B, L, Hkv, Kt)))
        tm = _mask(tok_mask)
        cm = _mask(chunk_mask)
        self.lib.oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(qs), dt, _ptr(ks), _ptr(idx_),
                            _ptr(sc), _ptr(w_), _ptr(do), B, L, Hq, Hkv, D, S, Kt,
                            float(sm_scale), float(sel_scale), int(bool(fold)), _wmode(weights),
                            _ptr(tm), _ptr(cm),
                            _ptr(out["dQ"]), _ptr(out["dK"]), _ptr(out["dV"]), _ptr(out["dQs"]),
                            _ptr(out["dKslc"]), _ptr(out["dw"]), _ptr(out["ds"]))
        return out

    # -- decode --------------------------------------------------------------------------
    def decode(self, q, qs, Kc, Vc, Kslc, S: int, K: int, sm_scale=None, sel_scale=None,
               score_dt: int = F32, weights: str = "stick"):
        """One new query per sequence at position ctx.  Returns dict(O, idx, score, w)."""
        q_, dt = _as_storage(q)
        qs_, _ = _as_storage(qs)
        kc, _ = _as_storage(Kc)
        vc, _ = _as_storage(Vc)
        B, Hq, D = q_.shape
        ctx, Hkv = kc.shape[1], kc.shape[2]
        ks = _f64(Kslc)
        assert ks.shape == (B, ctx // S, Hkv, D)
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(D)
        if sel_scale is None:
            sel_scale = 1.0 / math.sqrt(D)
        O = np.zeros((B, Hq, D))
        idx = np.full((B, Hkv, K), -1, np.int32)
        score = np.full((B, Hkv, K), -np.inf)
        w = np.zeros((B, Hkv, K))
        self.lib.oracle_decode(_ptr(q_), _ptr(qs_), _ptr(kc), _ptr(vc), dt, _ptr(ks), B, ctx, Hq,
                               Hkv, D, S, K, float(sm_scale), float(sel_scale), score_dt,
                               _wmode(weights), _ptr(O),
                               _ptr(idx), _ptr(score), _ptr(w))
        return dict(O=O, idx=idx, score=score, w=w)


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle build next to this file (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _default = Oracle(_LIB)
    return _default
