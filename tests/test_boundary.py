"""The product path and the oracle stay apart (CPU only): the binding refuses to run without
the HIP library, and no product source names the oracle."""
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "chunk_sparse_attention_amd")


def test_missing_library_fails_loudly(monkeypatch):
    """Without libhsa.so every entry point raises instead of computing anything another way."""
    from chunk_sparse_attention_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libhsa.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def test_product_sources_do_not_reach_the_oracle():
    """The package's Python, HIP and header files neither import nor include the oracle."""
    files = (glob.glob(os.path.join(PKG, "**", "*.py"), recursive=True)
             + glob.glob(os.path.join(PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*")))
    assert files
    pat = re.compile(r"^\s*(import\s+oracle|from\s+oracle|#\s*include\s*[<\"].*oracle)", re.M)
    for f in files:
        with open(f, errors="replace") as fh:
            text = fh.read()
        assert not pat.search(text), f
        assert "hsa_oracle" not in text, f
