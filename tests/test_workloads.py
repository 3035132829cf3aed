"""The seeded input generators: determinism, recipe, and bf16 rounding."""
import math

import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_torch_rne():
    g = np.random.default_rng(1)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 65504.0, 3.0e38, -3.0e38, 1e-40, np.inf, -np.inf],
                                 dtype=np.float32)])
    # ties: values exactly halfway between two bf16 numbers
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    assert np.isnan(W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]


def test_generators_are_deterministic_and_seeded():
    a = W.make_config(2, B=1, Hq=2, Hkv=2, Nq=64, Nk=64)
    b = W.make_config(2, B=1, Hq=2, Hkv=2, Nq=64, Nk=64)
    for n in ("q", "k", "v"):
        assert np.array_equal(a.tensors[n], b.tensors[n])
    assert not np.array_equal(a.tensors["q"], a.tensors["k"])
    c = W.make_config(3, B=1, Hq=2, Hkv=2, Nq=64, Nk=64)
    assert not np.array_equal(a.tensors["q"], c.tensors["q"])


def test_config_recipes():
    w1 = W.make_config(1)
    assert w1.tensors["q"].dtype == np.float32 and w1.tensors["q"].shape == (1, 1, 256, 64)
    assert not w1.causal and abs(w1.scale - 0.125) < 1e-15
    w3 = W.make_config(3, B=1, Hq=2, Hkv=2, Nq=1000, Nk=1000)
    # 1% of K rows per (b, h) scaled by 8 (exact in bf16): compare with the unscaled draw
    raw = W.normal_bf16_bits(W.rng(3, W.STREAM_K), (1, 2, 1000, 128))
    kv, rv = W.bf16_bits_to_f32(w3.tensors["k"]), W.bf16_bits_to_f32(raw)
    for h in range(2):
        rows = w3.outlier_rows[0, h]
        assert len(rows) == 10 and len(set(rows.tolist())) == 10
        assert np.array_equal(kv[0, h, rows], 8 * rv[0, h, rows])
        others = np.setdiff1d(np.arange(1000), rows)
        assert np.array_equal(kv[0, h, others], rv[0, h, others])
    assert w3.sample_rows.shape == (512, 3)
    assert len({tuple(r) for r in w3.sample_rows.tolist()}) == 512
    w4 = W.make_config(4, B=16, Hq=4, Hkv=1, Nk=2048, len_lo=100)
    assert w4.seqlens.dtype == np.int32 and w4.seqlens.min() >= 100 and w4.seqlens.max() <= 2048
    full = W.make_config.__wrapped__ if hasattr(W.make_config, "__wrapped__") else None
    assert full is None
    w5 = W.make_config(5, B=1, Hq=1, Hkv=1, Nq=64, Nk=64)
    assert "do" in w5.tensors and w5.causal


def test_full_decode_lengths_recipe():
    lens = W.cache_lengths(4, 16, 4096, 32768)
    assert lens.min() >= 4096 and lens.max() <= 32768
    assert np.array_equal(lens, W.cache_lengths(4, 16, 4096, 32768))


def test_values_are_normal():
    w = W.make_config(2, B=1, Hq=4, Hkv=4, Nq=2048, Nk=2048)
    x = w.values("q").astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_fp8_quantizer():
    """Per-tensor E4M3: power-of-two descale putting max|x| within 448, every
    value within half an E4M3 step (relative 2^-4 in the normal range), ties
    to the even code, saturation at 448."""
    import workloads as W
    x = np.random.Generator(np.random.PCG64(5)).standard_normal(20000).astype(np.float32)
    codes, s = W.fp8_quantize(x)
    assert math.log2(s) == int(math.log2(s)) and np.abs(x).max() / s <= 448
    back = W.e4m3_bits_to_f32(codes).astype(np.float64) * s
    normal = np.abs(x) / s >= 2.0 ** -6
    assert np.all(np.abs(back - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal] + 1e-12)
    assert np.all(np.abs(back - x)[~normal] <= 2.0 ** -10 * s + 1e-12)
    assert W.f32_to_e4m3_bits(np.array([1.0625]))[0] == 0x38     # tie between 1.0 (even) and 1.125
    assert W.f32_to_e4m3_bits(np.array([1.1875]))[0] == 0x3A     # tie between 1.125 and 1.25 (even)
    assert W.f32_to_e4m3_bits(np.array([1e6, -1e6])).tolist() == [0x7E, 0xFE]


def test_hash_values():
    """The index hash gives the same values from numpy and torch, on the 1/64
    grid in [-2, 2), with mean ~0, variance ~ that of U[-2, 2) and rows that are
    nearly uncorrelated (a linear hash fails the last check)."""
    import torch
    rows = np.arange(4096, dtype=np.int64)[:, None] + 12_000_000
    cols = np.arange(128, dtype=np.int64)[None, :]
    a = W.hash_values(rows, cols, 3)
    b = W.hash_values(torch.from_numpy(rows), torch.from_numpy(cols), 3).numpy()
    assert np.array_equal(a, b.astype(np.float64))
    assert np.array_equal(a * 64, np.round(a * 64)) and a.min() >= -2 and a.max() < 2
    assert abs(a.mean()) < 0.02 and abs(a.var() - 4 / 3) < 0.03
    c = np.corrcoef(a)[np.triu_indices(a.shape[0], 1)]
    assert np.abs(c).max() < 0.45 and np.abs(c).mean() < 0.1
    assert not np.array_equal(a, W.hash_values(rows, cols, 4))
