"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import exact_io_aware_16_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
CEIL_HEADER = os.path.join(ROOT, "include", "fa_ceilings.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(fa_\w+)\s*\(", text, flags=re.M)))


# FA_TEST_HOSTCHECK=<path of libfa_hostcheck.so>: run these checks against the
# C ABI layer built with AddressSanitizer/UndefinedBehaviorSanitizer over a
# stub launch layer (exact_io_aware_16_amd.build.build_hostcheck), with the
# sanitizer runtime preloaded; the success-path tests below then also run.
HOSTCHECK = os.environ.get("FA_TEST_HOSTCHECK")


@pytest.fixture(scope="module")
def lib():
    if HOSTCHECK:
        fa.load_library()   # torch's HIP runtime first, as the binding arranges
        h = ctypes.CDLL(HOSTCHECK)
        _declare(h)
        return h
    if not os.path.exists(fa.LIB_PATH):
        pytest.skip("libfa.so not built")
    return fa.load_library()


def _declare(h):
    """The argument types of every entry point, as the binding declares them."""
    ref = fa.load_library()
    for n in declared_functions():
        fn_ref, fn = getattr(ref, n), getattr(h, n)
        fn.restype, fn.argtypes = fn_ref.restype, fn_ref.argtypes
    h.fa_hostcheck_last_launch.restype = ctypes.c_char_p
    h.fa_hostcheck_last_launch.argtypes = [ctypes.POINTER(ctypes.c_longlong)]


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fa_fwd", "fa_fwd_fp8", "fa_bwd", "fa_decode", "fa_decode_chunk", "fa_decode_paged",
              "fa_decode_noalloc", "fa_bwd_workspace_bytes", "fa_decode_workspace_bytes",
              "fa_decode_chunk_workspace_bytes", "fa_decode_paged_workspace_bytes", "fa_abi_version",
              "fa_status_str"):
        assert n in names, names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} not exported"


def test_every_header_is_covered():
    """Each header under include/ belongs to a library the tests load."""
    assert sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")) == ["fa.h",
                                                                                             "fa_ceilings.h"]


def test_ceilings_library_exports_its_header():
    from exact_io_aware_16_amd import ceilings
    if not os.path.exists(ceilings.LIB_PATH):
        pytest.skip("libfa_ceilings.so not built")
    clib = ceilings.load_library()
    names = declared_functions(CEIL_HEADER)
    assert names == ["fa_ceil_device", "fa_ceil_hbm_read", "fa_ceil_hbm_read_lds", "fa_ceil_hbm_read_lds_bytes",
                     "fa_ceil_lds_read", "fa_ceil_mfma_bf16"], names
    for n in names:
        assert hasattr(clib, n), f"{n} not exported"
    # argument checks happen before anything is launched
    P = ctypes.c_void_p(0x1000)
    assert clib.fa_ceil_mfma_bf16(None, P, 1, 1, None) == 1
    assert clib.fa_ceil_mfma_bf16(P, P, 0, 1, None) == 1
    assert clib.fa_ceil_hbm_read(P, 17, P, 1, 8, None) == 1      # not a multiple of 16
    assert clib.fa_ceil_hbm_read(P, 4096, P, 1, 5, None) == 1    # loads in flight not 4/8/16
    assert clib.fa_ceil_lds_read(P, P, 4, 1, 1, None) == 1       # unknown mode
    # direct-to-LDS streaming read: shares rounded down to whole stages
    assert clib.fa_ceil_hbm_read_lds_bytes(1 << 30, 1024, 16) == (1 << 30)
    assert clib.fa_ceil_hbm_read_lds_bytes((1 << 20) + 5000, 4, 16) == 4 * 256 * 1024
    assert clib.fa_ceil_hbm_read_lds_bytes(1 << 20, 4, 12) == 0
    assert clib.fa_ceil_hbm_read_lds(P, 1 << 20, 4, 12, 2, 1, None) == 1     # stage size not 4/8/16 KB
    assert clib.fa_ceil_hbm_read_lds(P, 1 << 20, 4, 16, 5, 1, None) == 1     # stages not 2..4
    assert clib.fa_ceil_hbm_read_lds(P, 1 << 20, 4, 16, 2, 3, None) == 1     # policy not 0/1
    assert clib.fa_ceil_hbm_read_lds(P, 1 << 14, 4, 16, 2, 1, None) == 1     # less than a stage per wave
    assert clib.fa_ceil_hbm_read_lds(ctypes.c_void_p(0x1001), 1 << 20, 4, 16, 2, 1, None) == 1   # misaligned


def test_version_and_status_strings(lib):
    assert lib.fa_abi_version() == 1
    for s in range(9):
        assert lib.fa_status_str(s).decode().startswith(["FA_OK", "FA_ERR_NULL_PTR", "FA_ERR_SHAPE",
                                                           "FA_ERR_DTYPE", "FA_ERR_UNSUPPORTED",
                                                           "FA_ERR_WORKSPACE", "FA_ERR_HIP", "FA_ERR_ARG",
                                                           "FA_ERR_SCRATCH"][s])
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
    # float32 inputs give float32 gradients only: bf16 ones are refused on the host
    assert bwd(dtype=0, grad=1) == 3
    assert "float32" in lib.fa_status_str(3).decode()


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


def test_decode_noalloc_validation(lib):
    """Host checks of the no-allocation decode (all refused before any device work)."""
    def dec(seq=P, B=2, Hq=32, Hkv=8, Nmax=1024, d=128, dtype=1, scale=0.088):
        return lib.fa_decode_noalloc(P, P, P, seq, P, P, B, Hq, Hkv, Nmax, d, dtype, scale, N)
    assert dec(seq=N) == 1
    assert dec(Hq=30) == 2
    assert dec(Nmax=0) == 2
    assert dec(dtype=4) == 3
    assert dec(d=80) == 4
    assert dec(scale=-1.0) == 7
    # partial results beyond the fixed 64 MiB scratch: 4 query heads per K/V
    # head at d = 128 fit up to B * Hkv = 30465
    assert lib.fa_decode_workspace_bytes(1, 4 * 30466, 30466, 16, 128) > 64 << 20
    assert dec(B=1, Hq=4 * 30466, Hkv=30466, Nmax=16) == 8
    assert dec(B=2, Hq=4 * 30466, Hkv=30466, Nmax=16) == 8


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
              "fa_decode_noalloc", "fa_bwd_workspace_bytes",
              "fa_decode_workspace_bytes", "fa_decode_chunk_workspace_bytes", "fa_decode_paged_workspace_bytes",
              "fa_abi_version"):
        assert callable(getattr(fa, n))


def test_one_hip_runtime_in_the_process(lib):
    """The binding loads torch's HIP runtime first, so libfa shares it."""
    maps = open("/proc/self/maps").read().splitlines()
    hip = {line.split()[-1] for line in maps if "libamdhip64" in line}
    assert len(hip) == 1, hip


# ---------------------------------------------------------------------------
# the binding checks every tensor's shape and dtype against the others before
# anything reaches the C ABI (which sees only pointers and sizes); CPU tensors
# are enough, since these checks come before the device check
# ---------------------------------------------------------------------------

def test_binding_rejects_mismatched_tensors(lib):
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    z = lambda *shape, dt=bf: torch.zeros(*shape, dtype=dt)
    q, k, o, lse = z(2, 4, 8, 64), z(2, 2, 8, 64), z(2, 4, 8, 64), z(2, 4, 8, dt=f32)
    # forward
    with pytest.raises(ValueError, match="v has shape"):
        fa.prepare_fwd(q, k, z(2, 2, 9, 64), o, lse)
    with pytest.raises(ValueError, match="batch or head dimension"):
        fa.prepare_fwd(q, z(1, 2, 8, 64), z(1, 2, 8, 64), o, lse)
    with pytest.raises(ValueError, match="batch or head dimension"):
        fa.prepare_fwd(q, z(2, 2, 8, 128), z(2, 2, 8, 128), o, lse)
    with pytest.raises(TypeError, match="k is"):
        fa.prepare_fwd(q.float(), k, k, o.float(), lse)
    with pytest.raises(TypeError, match="o is"):
        fa.prepare_fwd(q, k, k, o.float(), lse)
    with pytest.raises(ValueError, match="o has shape"):
        fa.prepare_fwd(q, k, k, z(2, 4, 7, 64), lse)
    with pytest.raises(ValueError, match="lse has shape"):
        fa.prepare_fwd(q, k, k, o, z(2, 4, 7, dt=f32))
    with pytest.raises(TypeError, match="lse must be float32"):
        fa.prepare_fwd(q, k, k, o, z(2, 4, 8))
    with pytest.raises(ValueError, match="on the GPU"):   # well formed: stops at the device check
        fa.prepare_fwd(q, k, k, o, lse)
    # backward
    g32 = lambda t: torch.zeros(t.shape, dtype=f32)
    ws = z(1024, dt=torch.uint8)
    with pytest.raises(ValueError, match="dq has shape"):
        fa.prepare_bwd(q, k, k, o, o, lse, z(2, 4, 8, 32, dt=f32), g32(k), g32(k), ws)
    with pytest.raises(ValueError, match="dk has shape"):
        fa.prepare_bwd(q, k, k, o, o, lse, g32(q), g32(q), g32(k), ws)
    with pytest.raises(ValueError, match="dO has shape"):
        fa.prepare_bwd(q, k, k, o, z(2, 4, 9, 64), lse, g32(q), g32(k), g32(k), ws)
    with pytest.raises(TypeError, match="dO is"):
        fa.prepare_bwd(q, k, k, o, o.float(), lse, g32(q), g32(k), g32(k), ws)
    with pytest.raises(TypeError, match="share one dtype"):
        fa.prepare_bwd(q, k, k, o, o, lse, g32(q), g32(k).to(bf), g32(k), ws)
    with pytest.raises(TypeError, match="float32 gradients only"):
        fa.prepare_bwd(q.float(), k.float(), k.float(), o.float(), o.float(), lse, q, k, k, ws)
    with pytest.raises(ValueError, match="on the GPU"):
        fa.prepare_bwd(q, k, k, o, o, lse, g32(q), g32(k), g32(k), ws)
    # decode and chunk decode
    qd, kc, od = z(3, 8, 1, 128), z(3, 2, 100, 128), z(3, 8, 1, 128)
    sl, ld = torch.zeros(3, dtype=torch.int32), z(3, 8, dt=f32)
    with pytest.raises(ValueError, match="seqlens has shape"):
        fa.prepare_decode(qd, kc, kc, sl[:2], od, ld, ws)
    with pytest.raises(TypeError, match="seqlens must be int32"):
        fa.prepare_decode(qd, kc, kc, sl.long(), od, ld, ws)
    with pytest.raises(ValueError, match="one token per head"):
        fa.prepare_decode(z(3, 8, 2, 128), kc, kc, sl, z(3, 8, 2, 128), ld, ws)
    with pytest.raises(ValueError, match="lse has shape"):
        fa.prepare_decode(qd, kc, kc, sl, od, z(3, 4, dt=f32), ws)
    with pytest.raises(ValueError, match="v_cache has shape"):
        fa.prepare_decode(qd, kc, z(3, 2, 99, 128), sl, od, ld, ws)
    with pytest.raises(ValueError, match="on the GPU"):
        fa.prepare_decode(qd, kc, kc, sl, od, ld, ws)
    qc = z(3, 8, 4, 128)
    with pytest.raises(ValueError, match="lse has shape"):
        fa.prepare_decode_chunk(qc, kc, kc, sl, qc.clone(), ld, ws)
    with pytest.raises(ValueError, match="seqlens has shape"):
        fa.prepare_decode_chunk(qc, kc, kc, sl[:1], qc.clone(), z(3, 8, 4, dt=f32), ws)
    # paged decode
    kp, bt = z(10, 2, 64, 128), torch.zeros(3, 4, dtype=torch.int32)
    with pytest.raises(ValueError, match="block_table must be"):
        fa.prepare_decode_paged(qc, kp, kp, bt[:2], sl, qc.clone(), z(3, 8, 4, dt=f32), ws)
    with pytest.raises(TypeError, match="block_table must be int32"):
        fa.prepare_decode_paged(qc, kp, kp, bt.long(), sl, qc.clone(), z(3, 8, 4, dt=f32), ws)
    with pytest.raises(ValueError, match="head dimension"):
        fa.prepare_decode_paged(qc, z(10, 2, 64, 64), z(10, 2, 64, 64), bt, sl, qc.clone(), z(3, 8, 4, dt=f32), ws)
    with pytest.raises(ValueError, match="on the GPU"):
        fa.prepare_decode_paged(qc, kp, kp, bt, sl, qc.clone(), z(3, 8, 4, dt=f32), ws)
    # fp8 forward
    u8 = torch.uint8
    q8, k8 = z(2, 4, 8, 64, dt=u8), z(2, 2, 8, 64, dt=u8)
    with pytest.raises(ValueError, match="v8 has shape"):
        fa.prepare_fwd_fp8(q8, k8, z(2, 2, 7, 64, dt=u8), o, lse, 1.0, 1.0, 1.0)
    with pytest.raises(ValueError, match="lse has shape"):
        fa.prepare_fwd_fp8(q8, k8, k8, o, z(2, 4, dt=f32), 1.0, 1.0, 1.0)
    with pytest.raises(ValueError, match="on the GPU"):
        fa.prepare_fwd_fp8(q8, k8, k8, o, lse, 1.0, 1.0, 1.0)


# ---------------------------------------------------------------------------
# success paths through the stub launch layer (host-check build only): every
# argument check passes, the workspace layout is computed, and the launch the
# entry point would make is recorded instead of made
# ---------------------------------------------------------------------------

def _last(lib):
    out = (ctypes.c_longlong * 5)()
    kind = lib.fa_hostcheck_last_launch(out).decode()
    return kind, list(out)


@pytest.mark.skipif(not HOSTCHECK, reason="needs the host-check build (FA_TEST_HOSTCHECK)")
def test_hostcheck_success_paths(lib):
    ws, big = P, 1 << 40
    assert fwd(lib, B=2, Hq=8, Hkv=2, Nq=100, Nk=300, d=128, causal=1) == 0
    assert _last(lib) == ("fwd_bf16", [2, 8, 100, 128, 1])
    assert fwd(lib, dtype=0, d=64) == 0 and _last(lib)[0] == "fwd_f32"
    assert lib.fa_bwd(P, P, P, P, P, P, P, P, P, 1, 1, 4, 2, 64, 64, 128, 1, 0.088, 1, ws, big, N) == 0
    assert _last(lib) == ("bwd_bf16", [1, 4, 64, 128, 1])
    assert lib.fa_bwd(P, P, P, P, P, P, P, P, P, 0, 1, 4, 2, 64, 64, 64, 0, 0.125, 0, ws, big, N) == 0
    assert _last(lib)[0] == "bwd_f32"
    assert lib.fa_decode(P, P, P, P, P, P, 16, 32, 8, 32768, 128, 1, 0.088, ws, big, N) == 0
    assert _last(lib) == ("decode", [16, 32, 32768, 128, 1])
    assert lib.fa_decode(P, P, P, P, P, P, 3, 4, 4, 100, 64, 0, 0.125, ws, big, N) == 0
    assert _last(lib)[0] == "fwd_f32_lens"
    assert lib.fa_decode_chunk(P, P, P, P, P, P, 2, 32, 8, 8, 1024, 128, 1, 0.088, 1, ws, big, N) == 0
    assert _last(lib) == ("decode", [2, 256, 1024, 128, 8])   # Hq * Nq rows, causal chunk of 8
    assert lib.fa_decode_paged(P, P, P, P, P, P, P, 2, 32, 8, 4, 64, 64, 16, 128, 1, 0.088, 1, ws, big, N) == 0
    assert _last(lib) == ("decode_paged", [2, 128, 1024, 128, 4])
    assert lib.fa_fwd_fp8(P, P, P, P, P, 1, 4, 2, 77, 300, 128, 0.5, 0.25, 1.0, 0.088, 1, N) == 0
    assert _last(lib) == ("fwd_fp8", [1, 4, 77, 128, 1])
    # the no-allocation decode reaches its scratch lookup, which needs a GPU:
    # without one it reports FA_ERR_HIP (and launches nothing)
    assert lib.fa_decode_noalloc(P, P, P, P, P, P, 2, 8, 2, 100, 128, 1, 0.088, N) in (0, 6)
