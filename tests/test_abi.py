"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import exact_io_aware_16_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(fa_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.skip("libfa.so not built")
    return fa.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fa_fwd", "fa_fwd_fp8", "fa_bwd", "fa_decode", "fa_decode_chunk", "fa_decode_paged",
              "fa_bwd_workspace_bytes", "fa_decode_workspace_bytes", "fa_decode_chunk_workspace_bytes",
              "fa_decode_paged_workspace_bytes", "fa_abi_version", "fa_status_str"):
        assert n in names, names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} not exported"


def test_version_and_status_strings(lib):
    assert lib.fa_abi_version() == 1
    for s in range(8):
        assert lib.fa_status_str(s).decode().startswith(["FA_OK", "FA_ERR_NULL_PTR", "FA_ERR_SHAPE",
                                                           "FA_ERR_DTYPE", "FA_ERR_UNSUPPORTED",
                                                           "FA_ERR_WORKSPACE", "FA_ERR_HIP", "FA_ERR_ARG"][s])
    assert lib.fa_status_str(99).decode() == "unknown fa status"


def test_workspace_sizes(lib):
    w1 = lib.fa_bwd_workspace_bytes(2, 16, 4096, 128)
    w2 = lib.fa_bwd_workspace_bytes(2, 16, 8192, 128)
    assert w1 == 2 * (2 * 16 * 4096 * 4) and w2 == 2 * w1
    # decode partials do not grow with the cache length, only with the batch
    d1 = lib.fa_decode_workspace_bytes(16, 32, 8, 32768, 128)
    d2 = lib.fa_decode_workspace_bytes(16, 32, 8, 65536, 128)
    d3 = lib.fa_decode_workspace_bytes(32, 32, 8, 32768, 128)
    assert d1 == d2 and d3 > d1
    # far below the cache itself
    assert d1 < 16 * 8 * 32768 * 128 * 2 // 64
    assert lib.fa_bwd_workspace_bytes(0, 1, 1, 64) == 0
    assert lib.fa_decode_workspace_bytes(1, 3, 2, 64, 64) == 0   # Hq not a multiple of Hkv


# Fake, 16-byte-aligned, never-dereferenced addresses: every call below fails
# validation on the host, so nothing is launched and nothing is touched.
P = ctypes.c_void_p(0x1000)
N = ctypes.c_void_p(0)


def fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=64, dtype=1, scale=0.125, causal=0):
    return lib.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, dtype, scale, causal, N)


def test_fwd_validation(lib):
    assert fwd(lib, q=N) == 1
    assert fwd(lib, lse=N) == 1
    assert fwd(lib, B=0) == 2
    assert fwd(lib, Nk=0) == 2
    assert fwd(lib, Hq=3, Hkv=2) == 2
    assert fwd(lib, causal=1, Nq=9, Nk=8) == 2
    assert fwd(lib, B=1 << 16, Hq=1 << 10, Hkv=1, Nq=64, d=64) == 2   # > 2^31 elements
    assert fwd(lib, dtype=7) == 3
    assert fwd(lib, d=96) == 4
    assert fwd(lib, d=256) == 4
    assert fwd(lib, scale=0.0) == 7
    assert fwd(lib, scale=float("nan")) == 7
    assert fwd(lib, scale=float("inf")) == 7
    assert fwd(lib, q=ctypes.c_void_p(0x1008)) == 7   # misaligned


def test_bwd_validation(lib):
    def bwd(ws=P, wsb=1 << 20, grad=0, dtype=1, d=64, dq=P, Hq=2, Hkv=1):
        return lib.fa_bwd(P, P, P, P, P, P, dq, P, P, grad, 1, Hq, Hkv, 8, 8, d, dtype, 0.125, 1, ws, wsb, N)
    assert bwd(dq=N) == 1
    assert bwd(grad=5) == 3
    assert bwd(d=32) == 4
    assert bwd(Hq=3, Hkv=2) == 2
    assert bwd(ws=N) == 5
    assert bwd(wsb=4 * 8 * 2 - 1) == 5


def test_decode_validation(lib):
    def dec(seq=P, ws=P, wsb=1 << 24, d=128, Hq=32, Hkv=8, Nmax=1024):
        return lib.fa_decode(P, P, P, seq, P, P, 2, Hq, Hkv, Nmax, d, 1, 0.088, ws, wsb, N)
    assert dec(seq=N) == 1
    assert dec(Hq=30, Hkv=8) == 2
    assert dec(Nmax=0) == 2
    assert dec(d=80) == 4
    assert dec(ws=N) == 5
    need = lib.fa_decode_workspace_bytes(2, 32, 8, 1024, 128)
    assert dec(wsb=need - 1) == 5


def test_decode_chunk_validation(lib):
    def chunk(seq=P, ws=P, wsb=1 << 26, d=128, Hq=32, Hkv=8, Nq=8, Nmax=1024, causal=1):
        return lib.fa_decode_chunk(P, P, P, seq, P, P, 2, Hq, Hkv, Nq, Nmax, d, 1, 0.088, causal, ws, wsb, N)
    assert chunk(seq=N) == 1
    assert chunk(Hq=30, Hkv=8) == 2
    assert chunk(Nq=0) == 2
    assert chunk(Nq=65) == 2
    assert chunk(Nmax=0) == 2
    assert chunk(d=80) == 4
    assert chunk(ws=N) == 5
    need = lib.fa_decode_chunk_workspace_bytes(2, 32, 8, 8, 1024, 128)
    assert need > 0 and chunk(wsb=need - 1) == 5
    # one new token needs what decode needs; more tokens need more partial rows
    assert lib.fa_decode_chunk_workspace_bytes(2, 32, 8, 1, 1024, 128) == lib.fa_decode_workspace_bytes(2, 32, 8, 1024, 128)
    assert lib.fa_decode_chunk_workspace_bytes(2, 32, 8, 16, 1024, 128) > need
    assert lib.fa_decode_chunk_workspace_bytes(2, 32, 8, 65, 1024, 128) == 0


def test_decode_paged_validation(lib):
    def paged(table=P, ws=P, wsb=1 << 26, d=128, Hq=32, Hkv=8, Nq=1, pages=64, psz=64, maxp=16):
        return lib.fa_decode_paged(P, P, P, table, P, P, P, 2, Hq, Hkv, Nq, pages, psz, maxp, d, 1, 0.088, 1,
                                   ws, wsb, N)
    assert paged(table=N) == 1
    assert paged(Hq=30) == 2
    assert paged(Nq=65) == 2
    assert paged(pages=0) == 2
    assert paged(maxp=0) == 2
    assert paged(psz=48) == 4      # not a multiple of 32
    assert paged(d=96) == 4
    assert paged(ws=N) == 5
    need = lib.fa_decode_paged_workspace_bytes(2, 32, 8, 1, 128)
    assert need == lib.fa_decode_workspace_bytes(2, 32, 8, 1024, 128)
    assert paged(wsb=need - 1) == 5


def test_fwd_fp8_validation(lib):
    def f8(q=P, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=128, dq=1.0, dk=1.0, dv=1.0, scale=0.088, causal=0):
        return lib.fa_fwd_fp8(q, P, P, P, P, B, Hq, Hkv, Nq, Nk, d, dq, dk, dv, scale, causal, N)
    assert f8(q=N) == 1
    assert f8(B=0) == 2
    assert f8(Hq=3, Hkv=2) == 2
    assert f8(causal=1, Nq=9, Nk=8) == 2
    assert f8(d=96) == 4
    assert f8(dq=0.0) == 7
    assert f8(dv=float("nan")) == 7
    assert f8(dk=-1.0) == 7
    assert f8(q=ctypes.c_void_p(0x1008)) == 7


def test_binding_names_match_header():
    for n in ("fa_fwd", "fa_fwd_fp8", "fa_bwd", "fa_decode", "fa_decode_chunk", "fa_decode_paged",
              "fa_bwd_workspace_bytes",
              "fa_decode_workspace_bytes", "fa_decode_chunk_workspace_bytes", "fa_decode_paged_workspace_bytes",
              "fa_abi_version"):
        assert callable(getattr(fa, n))


def test_one_hip_runtime_in_the_process(lib):
    """The binding loads torch's HIP runtime first, so libfa shares it."""
    maps = open("/proc/self/maps").read().splitlines()
    hip = {line.split()[-1] for line in maps if "libamdhip64" in line}
    assert len(hip) == 1, hip
