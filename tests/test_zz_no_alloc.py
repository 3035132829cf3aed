"""fa_decode_noalloc on the GPU: the decode entry point that allocates nothing
(its partial results in the library's fixed per-device scratch) against
fa_decode with a caller workspace, through the C ABI.  Two calls in a row, the
second on a smaller input, so stale scratch contents from the first call are
in place; both must equal fa_decode bit for bit (same kernels, same work
split) and match the fp64 oracle within the bf16 tolerance."""
import numpy as np
import pytest

import exact_io_aware_16_amd as fa
import oracle
import workloads as W
from gpu_helpers import TOL_BF16, TOL_F32, announce, assert_close, to_device, to_host

pytestmark = pytest.mark.gpu


def both(q, k, v, lens, scale):
    import torch
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    ld = to_device(np.asarray(lens, dtype=np.int32))
    B, Hq = q.shape[0], q.shape[1]
    o1 = torch.empty_like(qd)
    l1 = torch.empty((B, Hq), dtype=torch.float32, device="cuda:0")
    fa.fa_decode(qd, kd, vd, ld, o1, l1, fa.decode_workspace(qd, kd), scale=scale)
    o2 = torch.full_like(qd, float("nan"))
    l2 = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda:0")
    fa.fa_decode_noalloc(qd, kd, vd, ld, o2, l2, scale=scale)
    torch.cuda.synchronize()
    return (o1, l1), (o2, l2)


def check(w, lens, tol):
    (o1, l1), (o2, l2) = both(w.tensors["q"], w.tensors["k"], w.tensors["v"], lens, w.scale)
    import torch
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "fa_decode_noalloc differs from fa_decode"
    O, L = oracle.ref_decode(w.values("q"), w.values("k"), w.values("v"), np.asarray(lens), scale=w.scale)
    assert_close("O", to_host(o2), O, tol)
    assert_close("LSE", to_host(l2), L, tol)


def test_noalloc_decode_matches_decode_twice_second_smaller():
    w = W.make_config(4, B=8, Nk=8192)
    lens = W.random_lengths(71, 8, 1, 8192)
    announce(f"no-alloc decode, call 1: B8 Hq32 Hkv8 Nmax8192 d128, lengths {lens.tolist()}")
    check(w, lens, TOL_BF16)
    w2 = W.random_case(72, 3, 8, 2, 1, 1000, 64)
    lens2 = np.array([1000, 0, 37], dtype=np.int32)
    announce("no-alloc decode, call 2 (smaller): B3 Hq8 Hkv2 Nmax1000 d64, lengths [1000, 0, 37]")
    check(w2, lens2, TOL_BF16)


def test_noalloc_decode_float32_needs_no_scratch():
    w = W.random_case(73, 2, 4, 1, 1, 300, 128, dtype="f32")
    announce("no-alloc decode, float32 B2 Hq4 Hkv1 Nmax300 d128")
    check(w, np.array([300, 17], dtype=np.int32), TOL_F32)


def test_noalloc_decode_refuses_shapes_beyond_its_scratch():
    import torch
    # 4 query heads per K/V head, d = 128: at most B * Hkv = 30465 fit; the
    # size check comes before any device work, so zero-size-looking tensors
    # are not touched
    B, Hkv, Hq = 1, 32768, 4 * 32768
    lib = fa.load_library()
    P = __import__("ctypes").c_void_p(0x1000)
    assert lib.fa_decode_noalloc(P, P, P, P, P, P, B, Hq, Hkv, 16, 128, 1, 0.088, None) == 8
    assert "FA_ERR_SCRATCH" in lib.fa_status_str(8).decode()
