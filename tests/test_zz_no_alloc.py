"""hsa_decode_noalloc: the decode step without a caller workspace (its scratch is a device
array inside the library).  Called through the C ABI with outputs the test allocates, it must
equal hsa_decode on the same inputs, bit for bit, on two calls in a row, the second with a
smaller input (fewer sequences, a shorter context, a smaller K), so that nothing the first
call left in the shared scratch reaches the second.  GPU only."""
from __future__ import annotations

import ctypes

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def _decode_noalloc(lib, prob, q, qs, Kc, Vc, Kslc, K_top):
    B, Hq, D = q.shape
    Hkv = qs.shape[1]
    dev = q.device
    O = torch.full((B, Hq, D), float("nan"), dtype=q.dtype, device=dev)
    idx = torch.full((B, Hkv, K_top), -7, dtype=torch.int32, device=dev)
    score = torch.full((B, Hkv, K_top), float("nan"), dtype=torch.float32, device=dev)
    w = torch.full((B, Hkv, K_top), float("nan"), dtype=torch.float32, device=dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = lib.hsa_decode_noalloc(ctypes.byref(prob), P(q), P(qs), P(Kc), P(Vc), P(Kslc), P(O),
                                P(idx), P(score), P(w),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.hsa_last_error()
    return O, idx, score, w


@pytest.mark.parametrize("generic", [False, True], ids=["default", "generic"])
def test_decode_noalloc_equals_decode(generic):
    import chunk_sparse_attention_amd as hsa
    from chunk_sparse_attention_amd import _lib
    assert torch.cuda.is_available()
    dev = torch.device("cuda:0")
    lib = _lib.lib()
    cases = [  # the second call is smaller in every dimension that sizes the scratch
        (workloads.Workload("noalloc_a", 4, 1 << 18, 16, 2, 64, 64, 8, torch.bfloat16), 31),
        (workloads.Workload("noalloc_b", 2, 64 * 9 + 3, 8, 1, 128, 64, 4, torch.bfloat16), 32),
    ]
    for wl, seed in cases:
        print("case", wl.name, "generic" if generic else "default", flush=True)
        x = workloads.make_decode_inputs(wl, seed=seed)
        q, qs, Kc, Vc = (x[k].to(dev) for k in ("q", "qs", "Kc", "Vc"))
        Kslc = hsa.pool(Kc)
        prob = hsa.problem(wl.B, wl.L, wl.Hq, wl.Hkv, wl.D, wl.K, wl.dtype, generic=generic)
        got = _decode_noalloc(lib, prob, q, qs, Kc, Vc, Kslc, wl.K)
        ref = hsa.decode(q, qs, Kc, Vc, Kslc, wl.K, generic=generic)
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "idx", "score", "w"), got, ref):
            assert torch.equal(a, b), (wl.name, name)
        assert bool((got[1] >= 0).all())
