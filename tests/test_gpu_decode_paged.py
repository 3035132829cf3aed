"""fa_decode_paged on the GPU: against the fp64 oracle on scattered pages
(bf16 and float32, causal chunks and single tokens, ragged lengths), bit for
bit against fa_decode_chunk on the contiguous cache the pages spell out (also
at the decode workload's full size), and with the pages the table never
reaches filled with NaN."""
import numpy as np
import pytest

import exact_io_aware_16_amd as fa
import oracle
import workloads as W
from gpu_helpers import TOL_BF16, TOL_F32, announce, assert_close, to_device, to_host

pytestmark = pytest.mark.gpu


def scatter(cache, page_size, num_pages, seed):
    """Contiguous [B, Hkv, max_pages*P, d] -> (pool [num_pages, Hkv, P, d], table
    [B, max_pages] int32) with the pages at seeded distinct positions; pool pages
    the table does not use hold other seeded values."""
    B, Hkv, N, d = cache.shape
    mp = N // page_size
    assert num_pages >= B * mp
    g = np.random.Generator(np.random.PCG64(seed))
    where = g.permutation(num_pages)[:B * mp].reshape(B, mp).astype(np.int32)
    pool = (g.integers(0, 1 << 16, size=(num_pages, Hkv, page_size, d)).astype(np.uint16) & np.uint16(0xBFFF)
            if cache.dtype == np.uint16 else g.standard_normal((num_pages, Hkv, page_size, d)).astype(np.float32))
    for b in range(B):
        for p in range(mp):
            pool[where[b, p]] = cache[b, :, p * page_size:(p + 1) * page_size]
    return pool, where


def run_paged(q, kp, vp, table, lens, scale, causal):
    o, lse = fa.decode_paged(to_device(q), to_device(kp), to_device(vp), to_device(table),
                             to_device(np.asarray(lens, dtype=np.int32)), causal=causal, scale=scale)
    return to_host(o), to_host(lse)


CASES = [
    # (B, Hq, Hkv, Nq, page_size, max_pages, extra pages, d, lengths)
    (3, 8, 2, 1, 32, 8, 5, 128, [256, 100, 0]),
    (2, 32, 8, 4, 64, 6, 3, 128, [384, 7]),
    (4, 4, 1, 8, 128, 3, 0, 64, [384, 129, 128, 8]),
    (2, 16, 2, 3, 32, 5, 10, 64, [1, 160]),
    (2, 4, 2, 2, 256, 2, 1, 128, [600, -3]),        # lengths clamped to the capacity
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}P{c[4]}x{c[5]}d{c[7]}")
def test_paged_against_oracle(case, dtype, causal):
    B, Hq, Hkv, Nq, P, mp, extra, d, lens = case
    w = W.random_case(P * mp + Hq, B, Hq, Hkv, Nq, P * mp, d, dtype=dtype)
    kp, table = scatter(w.tensors["k"], P, B * mp + extra, 5)
    vp, _ = scatter(w.tensors["v"], P, B * mp + extra, 5)
    announce(f"decode_paged {case} {dtype} causal={causal}")
    o, lse = run_paged(w.tensors["q"], kp, vp, table, lens, w.scale, causal)
    to_f = W.bf16_bits_to_f32 if dtype == "bf16" else (lambda x: x)
    O, L = oracle.ref_decode_paged(w.values("q"), to_f(kp), to_f(vp), table, np.array(lens), P, causal=causal,
                                   scale=w.scale)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert_close("O", o, O, tol)
    assert_close("LSE", lse, L, tol)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_paged_equals_contiguous_bit_for_bit(dtype):
    B, Hq, Hkv, Nq, P, mp, d = 5, 32, 8, 4, 64, 20, 128
    w = W.random_case(77, B, Hq, Hkv, Nq, P * mp, d, dtype=dtype)
    lens = W.random_lengths(77, B, 0, P * mp)
    kp, table = scatter(w.tensors["k"], P, B * mp + 7, 9)
    vp, _ = scatter(w.tensors["v"], P, B * mp + 7, 9)
    announce(f"decode_paged vs decode_chunk {dtype}, lengths {lens.tolist()}")
    qd, ld = to_device(w.tensors["q"]), to_device(lens)
    o1, l1 = fa.decode_chunk(qd, to_device(w.tensors["k"]), to_device(w.tensors["v"]), ld, causal=True)
    o2, l2 = fa.decode_paged(qd, to_device(kp), to_device(vp), to_device(table), ld, causal=True)
    assert np.array_equal(to_host(o1), to_host(o2)) and np.array_equal(to_host(l1), to_host(l2))


def test_unreached_pages_never_matter():
    B, Hq, Hkv, Nq, P, mp, d = 3, 8, 2, 2, 32, 6, 128
    w = W.random_case(78, B, Hq, Hkv, Nq, P * mp, d)
    lens = np.array([192, 33, 64], dtype=np.int32)
    kp, table = scatter(w.tensors["k"], P, B * mp + 4, 11)
    vp, _ = scatter(w.tensors["v"], P, B * mp + 4, 11)
    o1, l1 = run_paged(w.tensors["q"], kp, vp, table, lens, w.scale, True)
    used = {int(table[b, p]) for b in range(B) for p in range(-(-int(lens[b]) // P))}
    kp2, vp2, t2 = kp.copy(), vp.copy(), table.copy()
    for i in range(kp.shape[0]):
        if i not in used:
            kp2[i] = 0x7FC0
            vp2[i] = 0x7FC0
    t2[1, 3:] = 12345678    # past sequence 1's last page: never read (and clamped if it were)
    announce("decode_paged with NaN in every unreached page")
    o2, l2 = run_paged(w.tensors["q"], kp2, vp2, t2, lens, w.scale, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_decode_workload_paged_full_size():
    """The decode workload's cache (B16 Hkv8 Nmax32768 d128) in 64-key pages
    scattered over the pool: equal to the contiguous decode bit for bit."""
    w = W.make_config(4)
    P = 64
    kp, table = scatter(w.tensors["k"], P, w.B * (w.Nk // P), 13)
    vp, _ = scatter(w.tensors["v"], P, w.B * (w.Nk // P), 13)
    announce(f"decode_paged full size, lengths {w.seqlens.tolist()}")
    qd, ld = to_device(w.tensors["q"]), to_device(w.seqlens)
    o1, l1 = fa.decode(qd, to_device(w.tensors["k"]), to_device(w.tensors["v"]), ld)
    o2, l2 = fa.decode_paged(qd, to_device(kp), to_device(vp), to_device(table), ld)
    assert np.array_equal(to_host(o1), to_host(o2)[:, :, :1]) and np.array_equal(to_host(l1), to_host(l2)[:, :, 0])
