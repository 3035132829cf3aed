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


if __name__ == "__main__":
    build(verbose=True)
