"""Hierarchical Sparse Attention (HSA) for AMD Instinct MI355X (gfx950).

The operator lives in libhsa.so (hand-written HIP kernels behind the C ABI of
include/hsa.h); this package is its thin Python binding.  Importing the package does not
load the library; the first call does, and fails loudly if it has not been built.
"""
from .ops import (bwd, decode, decode_host_kv, decode_ragged, decode_shared,  # noqa: F401
                  fwd, fwd_layers, pool, pool_chunks, problem, select, timer_enable,
                  timer_read, workspace, workspace_size)

__all__ = ["select", "pool", "pool_chunks", "fwd", "fwd_layers", "bwd", "decode",
           "decode_host_kv", "decode_ragged", "decode_shared", "problem", "workspace",
           "workspace_size", "timer_enable", "timer_read"]
