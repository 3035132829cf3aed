"""fa_decode on the GPU against the fp64 oracle: the full GQA decode
configuration, ragged cache lengths, group sizes, and a poisoned cache tail."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import exact_io_aware_16_amd as fa
import oracle
import workloads as W
from gpu_helpers import TOL_BF16, TOL_F32, announce, assert_close, to_device, to_host

pytestmark = pytest.mark.gpu


def run_decode(q, k, v, lens, scale):
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    ld = to_device(np.asarray(lens, dtype=np.int32))
    o, lse = fa.decode(qd, kd, vd, ld, scale=scale)
    return to_host(o), to_host(lse)


def test_config4_gqa_decode_full():
    w = W.make_config(4)
    announce(f"config 4: decode B16 Hq32 Hkv8 Nmax32768 d128, lengths {w.seqlens.tolist()}")
    o, lse = run_decode(w.tensors["q"], w.tensors["k"], w.tensors["v"], w.seqlens, w.scale)
    O, L = oracle.ref_decode(w.values("q"), w.values("k"), w.values("v"), w.seqlens, scale=w.scale)
    assert_close("O", o, O, TOL_BF16)
    assert_close("LSE", lse, L, TOL_BF16)


CASES = [
    # (B, Hq, Hkv, Nmax, d, lengths)
    (4, 4, 1, 1024, 128, [1, 127, 128, 129]),
    (4, 8, 2, 2048, 64, [511, 512, 513, 2048]),
    (3, 32, 8, 4096, 128, [4096, 1000, 2]),
    (2, 32, 1, 700, 128, [700, 333]),          # MQA, 32 heads in one tile
    (2, 64, 1, 600, 64, [600, 5]),             # 64 heads per group: two head tiles
    (2, 6, 6, 1500, 128, [1500, 1499]),        # g = 1
    (3, 4, 2, 900, 128, [0, 900, 17]),         # empty sequence -> O = 0, LSE = -inf
    (2, 4, 2, 100, 128, [0, 0]),               # nothing to attend to anywhere
    (1, 1, 1, 1, 64, [1]),                     # a single key
    (2, 4, 1, 256, 128, [300, -5]),            # lengths clamped to [0, Nmax]
    (1, 8, 1, 32768, 128, [32768]),            # one long row shared by every wave
]


def test_decode_many_sequences_ragged():
    """More sequences than one wave's 64 lanes, zero lengths among them: the
    per-sequence stage counts are summed over several chunks of the batch."""
    B, Hq, Hkv, Nmax, d = 70, 4, 2, 300, 64
    lens = W.random_lengths(7, B, 0, Nmax)
    lens[::9] = 0
    w = W.random_case(70, B, Hq, Hkv, 1, Nmax, d)
    announce(f"decode B70 ragged lengths {lens.tolist()}")
    o, lse = run_decode(w.tensors["q"], w.tensors["k"], w.tensors["v"], lens, w.scale)
    O, L = oracle.ref_decode(w.values("q"), w.values("k"), w.values("v"), lens, scale=w.scale)
    assert_close("O", o, O, TOL_BF16)
    assert_close("LSE", lse, L, TOL_BF16)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}Hq{c[1]}Hkv{c[2]}N{c[3]}d{c[4]}")
def test_decode_shapes(case, dtype):
    B, Hq, Hkv, Nmax, d, lens = case
    w = W.random_case(Nmax + Hq, B, Hq, Hkv, 1, Nmax, d, dtype=dtype)
    announce(f"decode {case} {dtype}")
    o, lse = run_decode(w.tensors["q"], w.tensors["k"], w.tensors["v"], lens, w.scale)
    O, L = oracle.ref_decode(w.values("q"), w.values("k"), w.values("v"), np.array(lens), scale=w.scale)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert_close("O", o, O, tol)
    assert_close("LSE", lse, L, tol)


def test_poisoned_tail_is_never_read_into_the_result():
    B, Hq, Hkv, Nmax, d = 3, 8, 2, 2000, 128
    lens = np.array([1500, 1, 777], dtype=np.int32)
    w = W.random_case(11, B, Hq, Hkv, 1, Nmax, d)
    k, v = w.tensors["k"].copy(), w.tensors["v"].copy()
    o1, l1 = run_decode(w.tensors["q"], k, v, lens, w.scale)
    for b in range(B):
        k[b, :, lens[b]:] = 0x7FC0   # NaN
        v[b, :, lens[b]:] = 0x7F80   # +inf
    o2, l2 = run_decode(w.tensors["q"], k, v, lens, w.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.isfinite(o2).all()


def test_decode_is_deterministic():
    w = W.make_config(4, B=4, Nk=8192)
    o1, l1 = run_decode(w.tensors["q"], w.tensors["k"], w.tensors["v"], w.seqlens, w.scale)
    o2, l2 = run_decode(w.tensors["q"], w.tensors["k"], w.tensors["v"], w.seqlens, w.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_decode_equals_forward_with_one_query():
    w = W.random_case(5, 2, 8, 2, 1, 640, 128)
    lens = np.array([640, 640], dtype=np.int32)
    o_dec, l_dec = run_decode(w.tensors["q"], w.tensors["k"], w.tensors["v"], lens, w.scale)
    q, k, v = (to_device(w.tensors[n]) for n in ("q", "k", "v"))
    o_f, l_f = fa.fwd(q, k, v, causal=False, scale=w.scale)
    assert np.abs(o_dec - to_host(o_f)).max() <= 2e-2
    assert np.abs(l_dec - to_host(l_f)[:, :, 0]).max() <= 2e-2


def test_decode_workspace_needs_no_initialisation_and_is_reusable():
    """The caller's workspace needs no initialisation and may be reused: random
    bytes or all-ones before a call, then the same buffer for calls with other
    lengths and for a smaller shape, whose partial results and stage prefixes
    then sit where the previous call left other data."""
    import torch
    B, Hq, Hkv, Nmax, d = 5, 8, 2, 3000, 128
    w = W.random_case(21, B, Hq, Hkv, 1, Nmax, d)
    qd, kd, vd = (to_device(w.tensors[n]) for n in ("q", "k", "v"))
    ws = fa.decode_workspace(qd, kd)
    rng = np.random.default_rng(5)
    q, k, v = w.values("q"), w.values("k"), w.values("v")

    def check(lens, fill=None, qx=qd, kx=kd, vx=vd, ref=(q, k, v)):
        if fill is not None:
            ws.copy_(torch.from_numpy(fill).to(ws.device))
        announce(f"decode workspace reuse: lens {list(lens)}, fill {'kept' if fill is None else 'new'}")
        ld = to_device(np.asarray(lens, dtype=np.int32))
        o, lse = fa.decode(qx, kx, vx, ld, scale=w.scale, workspace=ws)
        O, L = oracle.ref_decode(*ref, np.asarray(lens), scale=w.scale)
        assert_close("O", to_host(o), O, TOL_BF16)
        assert_close("LSE", to_host(lse), L, TOL_BF16)

    n = ws.numel()
    check([3000, 1, 2999, 64, 1500], fill=rng.integers(0, 256, n, dtype=np.uint8))
    check([100, 3000, 0, 33, 2048])
    check([3000, 3000, 3000, 3000, 3000], fill=np.full(n, 0xFF, dtype=np.uint8))
    check([7, 8, 9, 10, 11])
    # a smaller batch and group in the same workspace
    q2, k2, v2 = q[:2, :4], k[:2, :1], v[:2, :1]
    check([2500, 900], qx=qd[:2, :4].contiguous(), kx=kd[:2, :1].contiguous(), vx=vd[:2, :1].contiguous(),
          ref=(q2, k2, v2))


def test_decode_cache_beyond_2gib():
    """One sequence of 12.5M cached keys at d = 128 (3.2 GB each for K and V):
    element offsets stay below 2^31 but byte offsets pass 2^31 (a signed
    32-bit byte offset would wrap).  The cache is built on the GPU from an
    integer hash of (key, column) and re-derived on the host, chunk by chunk,
    for the fp64 oracle of the 4 query heads."""
    import torch
    N, d, Hq, chunk = 12_500_000, 128, 4, 1 << 20
    announce(f"decode over a {N}-key cache (K and V {N * d * 2 / 2**30:.1f} GiB each)")
    dev = "cuda:0"
    k = torch.empty((1, 1, N, d), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    cols = torch.arange(d, device=dev, dtype=torch.int64)[None, :]
    for j0 in range(0, N, chunk):
        j = torch.arange(j0, min(N, j0 + chunk), device=dev, dtype=torch.int64)[:, None]
        k[0, 0, j0:j0 + j.shape[0]] = W.hash_values(j, cols, 1).to(torch.bfloat16)
        v[0, 0, j0:j0 + j.shape[0]] = W.hash_values(j, cols, 2).to(torch.bfloat16)
    q32 = np.random.Generator(np.random.PCG64(13)).standard_normal((1, Hq, 1, d)).astype(np.float32)
    q_bits = W.f32_to_bf16_bits(q32)
    qv = W.bf16_bits_to_f32(q_bits).astype(np.float64)[0, :, 0]          # [Hq, d]
    o, lse = fa.decode(to_device(q_bits), k, v, to_device(np.array([N], dtype=np.int32)))
    o, lse = to_host(o)[0, :, 0], to_host(lse)[0]
    del k, v
    torch.cuda.empty_cache()
    # oracle: the definition (ref_fwd) on each chunk of 2^20 keys, the chunks'
    # (O, LSE) pairs merged by merge_partials (pinned: a split merged equals
    # the unsplit result); the host never holds more than one chunk
    colsn = np.arange(d, dtype=np.int64)[None, :]
    pool = ThreadPoolExecutor(8)

    def gen(j, salt):   # the hash of one chunk of keys, its rows split over threads
        return np.concatenate(list(pool.map(lambda b: W.hash_values(b, colsn, salt), np.array_split(j, 8))))
    parts_o, parts_l = [], []
    for j0 in range(0, N, chunk):
        j = np.arange(j0, min(N, j0 + chunk), dtype=np.int64)[:, None]
        Oc, Lc = oracle.ref_fwd(qv[None, :, None, :], gen(j, 1)[None, None], gen(j, 2)[None, None], causal=False)
        parts_o.append(Oc[0, :, 0])
        parts_l.append(Lc[0, :, 0])
    pool.shutdown()
    O, L = oracle.merge_partials(np.stack(parts_o), np.stack(parts_l))
    assert_close("O", o, O, TOL_BF16)
    assert_close("LSE", lse, L, TOL_BF16)
