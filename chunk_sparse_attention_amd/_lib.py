"""ctypes view of libhsa.so (the C ABI declared in include/hsa.h).

Loading fails loudly when the library has not been built: there is no fallback path.
torch is imported first so that libhsa.so binds to the HIP runtime torch already loaded
(same soname), which lets torch's device pointers and streams be passed straight through.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the CDLL load, see module docstring)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhsa.so")

HSA_OK, HSA_ERR_INVALID_ARG, HSA_ERR_UNSUPPORTED, HSA_ERR_WORKSPACE, HSA_ERR_HIP = range(5)
HSA_F32, HSA_BF16 = 0, 1
HSA_OP_SELECT, HSA_OP_FWD, HSA_OP_BWD, HSA_OP_DECODE = range(4)
HSA_FLAG_GENERIC = 0x1
HSA_FLAG_SOFTMAX_WEIGHTS = 0x2
HSA_BWD_FOLD_KSLC = 0x1
HSA_BWD_AFTER_FWD = 0x2

EXPORTS = ("hsa_status_string", "hsa_last_error", "hsa_version", "hsa_workspace_size",
           "hsa_select", "hsa_fwd", "hsa_bwd", "hsa_decode", "hsa_decode_host_kv",
           "hsa_decode_ragged", "hsa_pool_chunks", "hsa_fwd_layers", "hsa_decode_shared",
           "hsa_decode_shared_host_kv", "hsa_timer_enable", "hsa_timer_read",
           "hsa_decode_noalloc")
# hsa_kernel_t: kernel classes of the timing aid
KERNEL_CLASSES = ("pool", "select", "tile_prep", "prep_ops", "fwd", "invidx", "bwd_p1", "bwd_p2",
                  "bwd_reduce", "decode_scan", "decode_attend", "fwd_token")


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("L", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("S", ctypes.c_int32),
                ("K", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("sel_scale", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class HsaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {_status_name(status)}: {detail}")


_lib: ctypes.CDLL | None = None


def _status_name(st: int) -> str:
    return {0: "HSA_OK", 1: "HSA_ERR_INVALID_ARG", 2: "HSA_ERR_UNSUPPORTED",
            3: "HSA_ERR_WORKSPACE", 4: "HSA_ERR_HIP"}.get(st, f"status {st}")


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m chunk_sparse_attention_amd.build`"
                           " (the HSA operator has no non-HIP implementation)")
    L = ctypes.CDLL(LIB_PATH)
    P, I, U, Z, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_float
    PP = ctypes.POINTER(Problem)
    L.hsa_status_string.restype = ctypes.c_char_p
    L.hsa_status_string.argtypes = [I]
    L.hsa_last_error.restype = ctypes.c_char_p
    L.hsa_last_error.argtypes = []
    L.hsa_version.restype = ctypes.c_char_p
    L.hsa_version.argtypes = []
    L.hsa_workspace_size.restype = I
    L.hsa_workspace_size.argtypes = [I, PP, ctypes.POINTER(Z)]
    L.hsa_select.restype = I
    L.hsa_select.argtypes = [PP, P, P, P, P, P, P, P, Z, P]
    L.hsa_fwd.restype = I
    L.hsa_fwd.argtypes = [PP, P, P, P, P, P, P, P, P, Z, P]
    L.hsa_bwd.restype = I
    L.hsa_bwd.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, U, P, Z, P]
    L.hsa_decode.restype = I
    L.hsa_decode.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, Z, P]
    L.hsa_decode_noalloc.restype = I
    L.hsa_decode_noalloc.argtypes = [PP, P, P, P, P, P, P, P, P, P, P]
    L.hsa_decode_host_kv.restype = I
    L.hsa_decode_host_kv.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, Z, P]
    L.hsa_decode_ragged.restype = I
    L.hsa_decode_ragged.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, Z, P]
    L.hsa_pool_chunks.restype = I
    L.hsa_pool_chunks.argtypes = [PP, P, P, P, I, P]
    L.hsa_fwd_layers.restype = I
    L.hsa_fwd_layers.argtypes = [PP, I, P, P, P, P, P, P, P, Z, P]
    L.hsa_decode_shared.restype = I
    L.hsa_decode_shared.argtypes = [PP, I, P, P, P, P, P, P, P]
    L.hsa_decode_shared_host_kv.restype = I
    L.hsa_decode_shared_host_kv.argtypes = [PP, I, P, P, P, P, P, P, P]
    L.hsa_timer_enable.restype = I
    L.hsa_timer_enable.argtypes = [I]
    L.hsa_timer_read.restype = I
    L.hsa_timer_read.argtypes = [I, ctypes.POINTER(I), ctypes.POINTER(ctypes.c_double)]
    _lib = L
    return L


def check(status: int, where: str) -> None:
    if status != HSA_OK:
        raise HsaError(status, where, lib().hsa_last_error().decode())
