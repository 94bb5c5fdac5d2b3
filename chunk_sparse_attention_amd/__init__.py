"""Hierarchical Sparse Attention (HSA) for AMD Instinct MI355X (gfx950).

The operator lives in libhsa.so (hand-written HIP kernels behind the C ABI of
include/hsa.h); this package is its thin Python binding.  Importing the package does not
load the library; the first call does, and fails loudly if it has not been built.
"""
from .ops import (bwd, decode, decode_host_kv, fwd, pool, problem, select,  # noqa: F401
                  timer_enable, timer_read, workspace, workspace_size)

__all__ = ["select", "pool", "fwd", "bwd", "decode", "decode_host_kv", "problem", "workspace",
           "workspace_size", "timer_enable", "timer_read"]
