"""fa_fwd_fp8 on the GPU against the fp64 oracle of exact attention on the
E4M3 inputs' values.

Tolerances (derived from the arithmetic; the pages fix none for FP8):
* The softmax weights of the second product are rounded to E4M3 (3 mantissa
  bits: relative error at most 2^-4), while the row sum adds the unrounded
  weights, so |O - O_exact| <= 2^-4 max_j |v_j| per row, plus the bf16
  rounding of O (2^-9 relative) and fp32 accumulation (~1e-5).  Random-input
  cases check that bound and rel-L2 <= 2^-4 (the same per-weight bound taken
  in norm: a statistical check, not a proof; a layout or masking mistake gives
  errors of order 1).
* LSE does not see the rounding of the weights: |LSE - LSE_exact| <= 2e-3
  (fp32 and the matrix cores' accumulation of the scores, ~2e-5 relative to
  sum |q_c k_c|).
* Integer-score cases (q and k entries in {-1, 0, 1}, scale * log2 e = 1)
  make every weight 2^8 * 2^(s - max) an exact E4M3 power of two, so only the
  bf16 rounding of O remains: max-abs <= 2^-8 max|O| + 1e-6.
"""
import math

import numpy as np
import pytest

import exact_io_aware_16_amd as fa
import oracle
import workloads as W
from gpu_helpers import announce, to_host

pytestmark = pytest.mark.gpu


def dev8(codes):
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to("cuda:0")


def run_fp8(q8, k8, v8, dq, dk, dv, causal, scale):
    o, lse = fa.fwd_fp8(dev8(q8), dev8(k8), dev8(v8), dq, dk, dv, causal=causal, scale=scale)
    return to_host(o), to_host(lse)


def check(name, o, lse, O, L, vmax, exact=False):
    err = np.abs(o - O).max()
    rel = np.linalg.norm(o - O) / max(np.linalg.norm(O), 1e-300)
    fin = np.isfinite(L)
    lerr = np.abs(lse[fin] - L[fin]).max() if fin.any() else 0.0
    print(f"  {name}: O max_abs={err:.3e} rel_l2={rel:.3e} (vmax {vmax:.3g}); LSE max_abs={lerr:.3e}", flush=True)
    assert np.array_equal(np.isneginf(lse), np.isneginf(L)), "LSE -inf pattern differs"
    assert lerr <= 2e-3, lerr
    if exact:
        assert err <= 2.0 ** -8 * np.abs(O).max() + 1e-6, err
    else:
        assert err <= (2.0 ** -4 + 2.0 ** -8) * vmax + 1e-5, err
        assert rel <= 2.0 ** -4, rel


SHAPES = [
    # (B, Hq, Hkv, Nq, Nk, d, causal)
    (1, 2, 2, 1, 1, 128, False),
    (1, 2, 1, 100, 100, 128, True),       # ragged blocks, GQA
    (2, 4, 2, 257, 257, 128, True),
    (1, 4, 4, 130, 333, 128, False),      # Nq != Nk
    (1, 2, 2, 77, 300, 128, True),        # bottom-right causal
    (2, 8, 2, 513, 513, 64, True),        # d = 64
    (1, 2, 1, 64, 1000, 64, False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}H{}x{}N{}x{}d{}{}".format(*s[:6], "c" if s[6] else ""))
def test_fp8_random_inputs(shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    w = W.random_case(sum(shape[:6]) + 900, B, Hq, Hkv, Nq, Nk, d, dtype="f32")
    f8 = W.to_fp8(w)
    (q8, dq), (k8, dk), (v8, dv) = f8["q"], f8["k"], f8["v"]
    sc = 1 / math.sqrt(d)
    announce(f"fp8 forward {shape}, descales {dq}, {dk}, {dv}")
    o, lse = run_fp8(q8, k8, v8, dq, dk, dv, causal, sc)
    O, L = oracle.ref_fwd_fp8(q8, k8, v8, dq, dk, dv, causal=causal, scale=sc)
    check("random", o, lse, O, L, np.abs(oracle.e4m3_value(v8) * dv).max())


@pytest.mark.parametrize("shape", [(1, 4, 2, 200, 200, 128, True), (2, 2, 2, 64, 640, 128, False),
                                   (1, 4, 1, 300, 300, 64, True)],
                         ids=lambda s: "B{}H{}x{}N{}x{}d{}{}".format(*s[:6], "c" if s[6] else ""))
def test_fp8_exact_weights(shape):
    """Scores are small integers and scale * log2 e = 1, so every weight is an
    exact E4M3 power of two: O must match to the bf16 rounding of the output."""
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    g = np.random.Generator(np.random.PCG64(sum(shape[:6])))

    def sparse_pm1(*shp):   # 3 entries of +-1 per row, the rest 0
        x = np.zeros(shp)
        flat = x.reshape(-1, shp[-1])
        for r in range(flat.shape[0]):
            idx = g.choice(shp[-1], 3, replace=False)
            flat[r, idx] = g.choice([-1.0, 1.0], 3)
        return x
    q8 = W.f32_to_e4m3_bits(sparse_pm1(B, Hq, Nq, d))
    k8 = W.f32_to_e4m3_bits(sparse_pm1(B, Hkv, Nk, d))
    v8, dv = W.fp8_quantize(g.standard_normal((B, Hkv, Nk, d)))
    sc = math.log(2.0)   # scale * log2(e) = 1
    announce(f"fp8 forward, exact weights {shape}")
    o, lse = run_fp8(q8, k8, v8, 1.0, 1.0, dv, causal, sc)
    O, L = oracle.ref_fwd_fp8(q8, k8, v8, 1.0, 1.0, dv, causal=causal, scale=sc)
    check("exact", o, lse, O, L, np.abs(oracle.e4m3_value(v8) * dv).max(), exact=True)


def test_fp8_llama_shape_sampled_rows():
    """The LLaMA-shaped causal workload (B2 H32 N8192 d128, 1% of K rows x8) in
    FP8 with per-tensor descales; 512 sampled rows against the oracle."""
    w = W.make_config(3)
    f8 = W.to_fp8(w)
    (q8, dq), (k8, dk), (v8, dv) = f8["q"], f8["k"], f8["v"]
    announce(f"fp8 forward B2 H32 N8192 d128 causal, descales {dq}, {dk}, {dv}")
    o, lse = run_fp8(q8, k8, v8, dq, dk, dv, True, w.scale)
    rows = w.sample_rows
    q = oracle.e4m3_value(q8) * dq
    k = oracle.e4m3_value(k8) * dk
    v = oracle.e4m3_value(v8) * dv
    O, L = oracle.ref_fwd_rows(q, k, v, rows, causal=True, scale=w.scale)
    og = np.stack([o[b, h, i] for b, h, i in rows])
    lg = np.array([lse[b, h, i] for b, h, i in rows])
    check("sampled", og, lg, O, L, np.abs(v).max())


def test_fp8_matches_bf16_path_on_the_same_values():
    """E4M3 values are exact in bf16, so the bf16 forward sees the same inputs:
    the two outputs differ only by the rounding of the weights (same bound)."""
    import torch
    B, Hq, Hkv, N, d = 2, 4, 2, 700, 128
    w = W.random_case(991, B, Hq, Hkv, N, N, d, dtype="f32")
    f8 = W.to_fp8(w)
    (q8, dq), (k8, dk), (v8, dv) = f8["q"], f8["k"], f8["v"]
    announce("fp8 vs bf16 forward on the same values")
    o8, l8 = run_fp8(q8, k8, v8, dq, dk, dv, True, None)
    vals = {n: torch.from_numpy((oracle.e4m3_value(c) * s).astype(np.float32)).to("cuda:0").to(torch.bfloat16)
            for n, (c, s) in f8.items()}
    ob, lb = fa.fwd(vals["q"], vals["k"], vals["v"], causal=True)
    ob, lb = to_host(ob), to_host(lb)
    vmax = np.abs(oracle.e4m3_value(v8) * dv).max()
    assert np.abs(o8 - ob).max() <= (2.0 ** -4 + 2.0 ** -7) * vmax
    assert np.abs(l8 - lb).max() <= 2e-3
