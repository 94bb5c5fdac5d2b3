"""Host-side checks of libhsa.so's C ABI (CPU only: no kernel is launched).

The library must load, export every function include/hsa.h declares, and reject invalid
arguments with the documented status before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hsa.h")
LIB = os.path.join(ROOT, "chunk_sparse_attention_amd", "libhsa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libhsa.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hsa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    from chunk_sparse_attention_amd import _lib
    lib = _lib.lib()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    from chunk_sparse_attention_amd import _lib
    lib = _lib.lib()
    assert lib.hsa_status_string(0) == b"HSA_OK"
    assert lib.hsa_status_string(3) == b"HSA_ERR_WORKSPACE"
    assert lib.hsa_version().decode().count(".") == 2


def _prob(**kw):
    from chunk_sparse_attention_amd import _lib
    base = dict(B=1, L=1024, Hq=4, Hkv=1, D=64, S=64, K=4, sm_scale=0.0, sel_scale=0.0, dtype=1,
                flags=0)
    base.update(kw)
    return _lib.Problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 1), (dict(L=0), 1), (dict(K=0), 1), (dict(Hq=6, Hkv=4), 2),
    (dict(Hq=64, Hkv=2), 2), (dict(D=96), 2), (dict(S=32), 2), (dict(K=17), 2),
    (dict(dtype=7), 2), (dict(sm_scale=float("inf")), 1), (dict(L=1 << 30, K=4), 2),
])
def test_workspace_size_validation(kw, status):
    from chunk_sparse_attention_amd import _lib
    lib = _lib.lib()
    n = ctypes.c_size_t(123)
    st = lib.hsa_workspace_size(_lib.HSA_OP_FWD, ctypes.byref(_prob(**kw)), ctypes.byref(n))
    assert st == status, lib.hsa_last_error()
    assert lib.hsa_last_error() != b""


def test_workspace_sizes_positive_where_needed():
    from chunk_sparse_attention_amd import _lib
    lib = _lib.lib()
    n = ctypes.c_size_t(0)
    p = _prob(B=2, L=16384, Hq=16, Hkv=2, K=8)
    assert lib.hsa_workspace_size(_lib.HSA_OP_BWD, ctypes.byref(p), ctypes.byref(n)) == 0
    assert n.value > 2 * 16384 * 2 * 8 * 4
    assert lib.hsa_workspace_size(_lib.HSA_OP_DECODE, ctypes.byref(p), ctypes.byref(n)) == 0
    assert n.value > 0
    assert lib.hsa_workspace_size(9, ctypes.byref(p), ctypes.byref(n)) == 1


def test_backward_chunk_limit():
    """The backward takes up to 32767 chunks (its inverse index splits the chunks into parts
    of 16384 past that many); beyond, HSA_ERR_UNSUPPORTED."""
    from chunk_sparse_attention_amd import _lib
    lib = _lib.lib()
    n = ctypes.c_size_t(0)
    for nC, status in ((16384, 0), (16385, 0), (32767, 0), (32768, 2)):
        p = _prob(L=64 * nC, K=2)
        assert lib.hsa_workspace_size(_lib.HSA_OP_BWD, ctypes.byref(p), ctypes.byref(n)) == status, nC
    assert b"32767" in lib.hsa_last_error()


def test_entry_points_reject_before_launch():
    """NULL / misaligned pointers and missing workspace are reported without any launch."""
    from chunk_sparse_attention_amd import _lib
    lib = _lib.lib()
    p = _prob()
    fake = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
    odd = ctypes.c_void_p(0x10002)
    st = lib.hsa_select(None, fake, fake, fake, fake, fake, fake, None, 0, None)
    assert st == 1
    st = lib.hsa_select(ctypes.byref(p), fake, None, fake, fake, fake, fake, None, 0, None)
    assert st == 1 and b"K is NULL" in lib.hsa_last_error()
    st = lib.hsa_fwd(ctypes.byref(p), odd, fake, fake, fake, fake, fake, None, None, 0, None)
    assert st == 1 and b"aligned" in lib.hsa_last_error()
    st = lib.hsa_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, odd, None, 0, None)
    assert st == 1 and b"lse is not 4-byte aligned" in lib.hsa_last_error()
    st = lib.hsa_bwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, None, fake,
                     fake, fake, fake, fake, None, 1, None, 0, None)
    assert st == 3, lib.hsa_last_error()
    st = lib.hsa_bwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, odd, fake,
                     fake, fake, fake, fake, None, 1, fake, 1 << 40, None)
    assert st == 1 and b"lse is not 4-byte aligned" in lib.hsa_last_error()
    st = lib.hsa_bwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                     fake, fake, fake, fake, None, 0x80, fake, 1 << 40, None)
    assert st == 1 and b"flags" in lib.hsa_last_error()
    st = lib.hsa_decode(ctypes.byref(_prob(D=80)), fake, fake, fake, fake, fake, fake, fake, None,
                        fake, fake, 1 << 30, None)
    assert st == 2
    st = lib.hsa_decode_ragged(ctypes.byref(_prob()), None, fake, fake, fake, fake, fake, fake,
                               fake, None, fake, fake, 1 << 30, None)
    assert st == 1 and b"ctx_lens is NULL" in lib.hsa_last_error()
    st = lib.hsa_pool_chunks(ctypes.byref(_prob()), fake, fake, fake, 0, None)
    assert st == 1 and b"n_ids" in lib.hsa_last_error()
    st = lib.hsa_fwd_layers(ctypes.byref(_prob()), 0, fake, fake, fake, fake, fake, fake, fake,
                            1 << 30, None)
    assert st == 1 and b"n_layers" in lib.hsa_last_error()
    st = lib.hsa_decode_shared(ctypes.byref(_prob()), 0, fake, fake, fake, fake, fake, fake, None)
    assert st == 1 and b"n_layers" in lib.hsa_last_error()
    st = lib.hsa_decode_shared_host_kv(ctypes.byref(_prob()), 0, fake, fake, fake, fake, fake,
                                       fake, None)
    assert st == 1 and b"n_layers" in lib.hsa_last_error()
    st = lib.hsa_decode_shared_host_kv(ctypes.byref(_prob()), 1, fake, None, fake, fake, fake,
                                       fake, None)
    assert st == 1 and b"Kcache" in lib.hsa_last_error()
    bad = _prob()
    bad.flags = 0x4  # no such problem flag
    st = lib.hsa_select(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, None, 0, None)
    assert st == 1 and b"unknown problem flags" in lib.hsa_last_error()
    st = lib.hsa_decode_host_kv(ctypes.byref(_prob(D=80)), fake, fake, fake, fake, fake, fake,
                                fake, None, fake, fake, 1 << 30, None)
    assert st == 2
    st = lib.hsa_decode_host_kv(ctypes.byref(_prob()), fake, fake, None, fake, fake, fake, fake,
                                None, fake, fake, 1 << 30, None)
    assert st == 1 and b"Kcache is NULL" in lib.hsa_last_error()


def test_binding_refuses_cpu_tensors():
    import torch
    import chunk_sparse_attention_amd as hsa
    x = torch.zeros((1, 128, 1, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        hsa.select(x, x, 4)


def test_binding_host_kv_needs_pinned_caches():
    """The host-cache decode takes pinned host tensors only (checked before any GPU call)."""
    import torch
    import chunk_sparse_attention_amd as hsa
    x = torch.zeros((1, 128, 1, 64), dtype=torch.bfloat16)
    q = torch.zeros((1, 4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="pinned host tensor"):
        hsa.decode_host_kv(q, q[:, :1], x, x, x[:, :2], 2)


def test_kernel_timer_without_launches():
    """The timing aid records nothing until a launch happens and validates its class."""
    from chunk_sparse_attention_amd import _lib
    L = _lib.lib()
    assert L.hsa_timer_enable(1) == _lib.HSA_OK
    n, ms = ctypes.c_int(-1), ctypes.c_double(-1.0)
    for k in range(len(_lib.KERNEL_CLASSES)):
        assert L.hsa_timer_read(k, ctypes.byref(n), ctypes.byref(ms)) == _lib.HSA_OK
        assert (n.value, ms.value) == (0, 0.0)
    assert L.hsa_timer_read(len(_lib.KERNEL_CLASSES), ctypes.byref(n),
                            ctypes.byref(ms)) == _lib.HSA_ERR_INVALID_ARG
    assert L.hsa_timer_read(-1, ctypes.byref(n), ctypes.byref(ms)) == _lib.HSA_ERR_INVALID_ARG
    assert L.hsa_timer_read(0, None, ctypes.byref(ms)) == _lib.HSA_ERR_INVALID_ARG
    assert L.hsa_timer_enable(0) == _lib.HSA_OK
    with open(HEADER) as fh:
        text = fh.read()
    for i, name in enumerate(_lib.KERNEL_CLASSES):
        assert f"HSA_KERNEL_{name.upper()} = {i}," in text


def test_decode_noalloc_refuses_oversized_scratch():
    """hsa_decode_noalloc keeps its scratch in a 4 MiB device array: a problem that needs more
    is refused with HSA_ERR_UNSUPPORTED before anything touches the GPU."""
    from chunk_sparse_attention_amd import _lib
    lib = _lib.lib()
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: the size check comes first
    # 8 bytes * B * Hkv * one scan block * K = 64 MiB of candidate keys
    p = _prob(B=1 << 16, L=64, Hq=8, Hkv=8, K=16)
    st = lib.hsa_decode_noalloc(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, None,
                                fake, None)
    assert st == 2 and b"scratch" in lib.hsa_last_error(), lib.hsa_last_error()
    st = lib.hsa_decode_noalloc(None, fake, fake, fake, fake, fake, fake, fake, None, fake, None)
    assert st == 1
