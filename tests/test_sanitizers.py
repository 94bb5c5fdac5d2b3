"""The CPU oracle and the library's host code under AddressSanitizer and UndefinedBehavior-
Sanitizer (CPU only; no kernel is launched).

  * hsa_oracle.c is rebuilt with gcc -fsanitize=address,undefined and every oracle pin runs
    on that build, in a child process that preloads gcc's ASan runtime;
  * libhsa.so is rebuilt with the sanitizers on its host code only (device code cannot take
    them) and the ABI tests, which drive the argument validation, run on that build in a
    child process that preloads clang's ASan runtime.
Any sanitizer report aborts the child (halt_on_error), which fails the test.  Leak checking
is off: the Python interpreter itself is not instrumented.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunk_sparse_attention_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.slow

ENV = dict(ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _child(code: str, preload: str, *args) -> subprocess.CompletedProcess:
    env = dict(os.environ, LD_PRELOAD=preload, **ENV)
    return subprocess.run([sys.executable, "-c", textwrap.dedent(code), *args], env=env,
                          capture_output=True, text=True, timeout=900)


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-Wall",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-o", lib,
                    os.path.join(ROOT, "oracle", "hsa_oracle.c"), "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    r = _child(f"""
        import sys
        sys.path[:0] = [{ROOT!r}, {os.path.join(ROOT, "tests")!r}]
        import oracle, pins
        orc = oracle.Oracle(sys.argv[1])
        for p in pins.ALL_PINS:
            p(orc)
        print("pins ok", len(pins.ALL_PINS))
        """, asan, lib)
    assert r.returncode == 0 and "pins ok" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_validation_under_asan_ubsan(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden",
             "-mcode-object-version=5", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
             "-Xarch_host", "-fno-omit-frame-pointer"]
    # the sanitizers apply to the host pass only
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    procs, objs = [], []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *flags, *san, "-c", src, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out.decode(errors="replace")[-3000:]
    lib = str(tmp_path / "libhsa_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan", *san,
                    "-o", lib, *objs], check=True, capture_output=True)
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    assert rt, "clang's ASan runtime not found"
    r = _child(f"""
        import sys
        sys.path[:0] = [{ROOT!r}, {os.path.join(ROOT, "tests")!r}]
        from chunk_sparse_attention_amd import _lib
        _lib.LIB_PATH = sys.argv[1]
        assert _lib.lib()._name == sys.argv[1]
        import pytest
        sys.exit(pytest.main(["-q", "-p", "no:cacheprovider",
                              {os.path.join(ROOT, "tests", "test_abi.py")!r}]))
        """, rt[0], lib)
    assert r.returncode == 0 and "passed" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
