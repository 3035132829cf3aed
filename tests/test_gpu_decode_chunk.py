"""fa_decode_chunk on the GPU against the fp64 oracle: Nq new tokens per head
against a KV cache whose last Nq keys are theirs, causal to each sequence's own
length (or not), ragged lengths including sequences shorter than the chunk,
several head tiles per K/V head, float32 and bfloat16, and the decode-shaped
cache at full size (Nq = 8) on sampled sequences."""
import numpy as np
import pytest

import exact_io_aware_16_amd as fa
import oracle
import workloads as W
from gpu_helpers import TOL_BF16, TOL_F32, announce, assert_close, to_device, to_host

pytestmark = pytest.mark.gpu


def run_chunk(q, k, v, lens, scale, causal):
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    ld = to_device(np.asarray(lens, dtype=np.int32))
    o, lse = fa.decode_chunk(qd, kd, vd, ld, causal=causal, scale=scale)
    return to_host(o), to_host(lse)


CASES = [
    # (B, Hq, Hkv, Nq, Nmax, d, lengths)
    (3, 8, 2, 4, 1024, 128, [1024, 500, 3]),      # last sequence shorter than the chunk
    (2, 32, 8, 8, 2048, 128, [2048, 1111]),       # g * Nq = 32: one head tile
    (2, 32, 8, 16, 700, 64, [700, 40]),           # g * Nq = 64: two head tiles
    (2, 4, 1, 64, 600, 128, [600, 64]),           # Nq = 64, 8 head tiles; token 0 of b=1 sees key 0 only
    (2, 4, 2, 5, 300, 64, [300, 0]),              # an empty sequence
    (2, 6, 6, 3, 100, 128, [2, 100]),             # g = 1; len 2 < Nq 3
    (1, 8, 1, 7, 32768, 128, [32768]),            # one long row shared by every wave
    (4, 4, 1, 2, 256, 128, [300, -5, 1, 2]),      # lengths clamped to [0, Nmax]
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}N{c[4]}d{c[5]}")
def test_chunk_shapes(case, dtype, causal):
    B, Hq, Hkv, Nq, Nmax, d, lens = case
    w = W.random_case(Nmax + Hq + Nq, B, Hq, Hkv, Nq, Nmax, d, dtype=dtype)
    announce(f"decode_chunk {case} {dtype} causal={causal}")
    o, lse = run_chunk(w.tensors["q"], w.tensors["k"], w.tensors["v"], lens, w.scale, causal)
    O, L = oracle.ref_decode_chunk(w.values("q"), w.values("k"), w.values("v"), np.array(lens), causal=causal,
                                   scale=w.scale)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert_close("O", o, O, tol)
    assert_close("LSE", lse, L, tol)


def test_one_token_chunk_is_decode_bit_for_bit():
    B, Hq, Hkv, Nmax, d = 5, 32, 8, 3000, 128
    lens = W.random_lengths(31, B, 0, Nmax)
    w = W.random_case(31, B, Hq, Hkv, 1, Nmax, d)
    announce(f"decode_chunk Nq=1 vs decode, lengths {lens.tolist()}")
    qd, kd, vd = to_device(w.tensors["q"]), to_device(w.tensors["k"]), to_device(w.tensors["v"])
    ld = to_device(lens)
    o1, l1 = fa.decode(qd, kd, vd, ld)
    for causal in (True, False):
        o2, l2 = fa.decode_chunk(qd, kd, vd, ld, causal=causal)
        assert np.array_equal(to_host(o1), to_host(o2)) and np.array_equal(to_host(l1), to_host(l2)[:, :, 0])


def test_poisoned_tail_is_never_read_into_the_result():
    B, Hq, Hkv, Nq, Nmax, d = 3, 8, 2, 6, 2000, 128
    lens = np.array([1500, 4, 777], dtype=np.int32)
    w = W.random_case(12, B, Hq, Hkv, Nq, Nmax, d)
    k, v = w.tensors["k"].copy(), w.tensors["v"].copy()
    o1, l1 = run_chunk(w.tensors["q"], k, v, lens, w.scale, True)
    for b in range(B):
        k[b, :, lens[b]:] = 0x7FC0   # NaN
        v[b, :, lens[b]:] = 0x7FC0
    announce("decode_chunk poisoned tail")
    o2, l2 = run_chunk(w.tensors["q"], k, v, lens, w.scale, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_decode_shaped_cache_full_size_sampled_sequences():
    """B16 Hq32 Hkv8 Nmax32768 d128 with the decode workload's cache and seeded
    lengths, 8 new tokens per head; the oracle checks three whole sequences."""
    w = W.make_config(4, Nq=8)
    announce(f"decode_chunk B16 Hq32 Hkv8 Nq8 Nmax32768 d128, lengths {w.seqlens.tolist()}")
    o, lse = run_chunk(w.tensors["q"], w.tensors["k"], w.tensors["v"], w.seqlens, w.scale, True)
    q = w.values("q")
    for b in (0, 7, 15):
        kb = W.bf16_bits_to_f32(w.tensors["k"][b:b + 1])
        vb = W.bf16_bits_to_f32(w.tensors["v"][b:b + 1])
        O, L = oracle.ref_decode_chunk(q[b:b + 1], kb, vb, w.seqlens[b:b + 1], causal=True, scale=w.scale)
        assert_close(f"O[b={b}]", o[b:b + 1], O, TOL_BF16)
        assert_close(f"LSE[b={b}]", lse[b:b + 1], L, TOL_BF16)
