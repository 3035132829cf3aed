"""Build libfa.so (the HIP kernels and the C ABI) and libfa_ceilings.so (the
measured-ceiling kernels the benchmark reports beside the attention rows) for
gfx950, in-tree.

Usage: ``python -m exact_io_aware_16_amd.build`` or ``build()`` from Python.
Each .hip source is compiled to an object in parallel, then linked into
``exact_io_aware_16_amd/libfa.so`` and ``exact_io_aware_16_amd/libfa_ceilings.so``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
OUT = os.path.join(PKG, "libfa.so")
OUT_CEILINGS = os.path.join(PKG, "libfa_ceilings.so")
BUILD = os.path.join(PKG, "_build")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_fwd_fp8.hip", "fa_decode.hip", "fa_bwd.hip"]
CEILING_SOURCES = ["fa_ceilings.hip"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(out)} failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every kernel source and link libfa.so and libfa_ceilings.so;
    returns the path of libfa.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEILING_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], OUT)
    _link([objs[s] for s in CEILING_SOURCES], OUT_CEILINGS)
    if verbose:
        print(f"built {OUT} and {OUT_CEILINGS}")
    return OUT


OUT_HOSTCHECK = os.path.join(PKG, "libfa_hostcheck.so")


def build_hostcheck(verbose: bool = False) -> str:
    """The C ABI layer (fa_api.hip) with a stub launch layer (host_stubs.cpp)
    that launches nothing, with AddressSanitizer and UndefinedBehaviorSanitizer
    on the host code: libfa_hostcheck.so, for tests/test_abi.py run as
    ``FA_TEST_HOSTCHECK=<path> LD_PRELOAD=<asan runtime> pytest tests/test_abi.py``.
    Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    objs = []
    for src in ("fa_api.hip", "host_stubs.cpp"):
        obj = os.path.join(BUILD, "hostcheck_" + os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *FLAGS, *san, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        objs.append(obj)
    tmp = OUT_HOSTCHECK + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-fsanitize=address", "-fsanitize=undefined",
           "-shared-libsan", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of libfa_hostcheck.so failed:\n{r.stderr}")
    os.replace(tmp, OUT_HOSTCHECK)
    if verbose:
        print(f"built {OUT_HOSTCHECK}")
    return OUT_HOSTCHECK


if __name__ == "__main__":
    import sys
    if "--hostcheck" in sys.argv:
        build_hostcheck(verbose=True)
    else:
        build(verbose=True)
