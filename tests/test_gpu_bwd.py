"""fa_bwd on the GPU against the fp64 oracle gradients.

The GPU backward consumes what fa_fwd produced (O in the input dtype and the
float32 row logsumexp), as a training step would; the oracle differentiates the
exact definition.  Tolerances: bf16 inputs max-abs 2e-2 and rel-L2 5e-3 on dQ,
dK, dV (float32 gradients); fp32 inputs max-abs 1e-5."""
import numpy as np
import pytest

import exact_io_aware_16_amd as fa
import oracle
import workloads as W
from gpu_helpers import TOL_BF16, TOL_F32, announce, assert_close, to_device, to_host

pytestmark = pytest.mark.gpu


def run_fwd_bwd(w, causal, grad_dtype=None):
    import torch
    q, k, v, do = (to_device(w.tensors[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=causal, scale=w.scale)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=causal, scale=w.scale, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return to_host(o), to_host(lse), to_host(dq), to_host(dk), to_host(dv)


def test_config5_fwd_bwd_full():
    w = W.make_config(5)
    announce("config 5: B2 H16 N4096 d128 bf16 causal fwd+bwd (full fp64 oracle)")
    o, lse, dq, dk, dv = run_fwd_bwd(w, True)
    q, k, v, do = (w.values(n) for n in ("q", "k", "v", "do"))
    O, L = oracle.ref_fwd(q, k, v, causal=True, scale=w.scale)
    assert_close("O", o, O, TOL_BF16)
    assert_close("LSE", lse, L, TOL_BF16)
    dQ, dK, dV = oracle.ref_bwd(q, k, v, do, causal=True, scale=w.scale)
    assert_close("dQ", dq, dQ, TOL_BF16)
    assert_close("dK", dk, dK, TOL_BF16)
    assert_close("dV", dv, dV, TOL_BF16)


def test_gqa_training_shape_fwd_bwd():
    """Grouped heads at a training shape (B2 Hq32 Hkv8 N4096 d128, causal, the
    config-5 recipe with 4 query heads per K/V head): dK and dV of a K/V head
    are the sums over its group, formed without atomics.  The fp64 oracle
    checks batch 0 whole (32 query heads, 8 K/V heads)."""
    w = W.make_config(5, Hq=32, Hkv=8)
    announce("GQA fwd+bwd B2 Hq32 Hkv8 N4096 d128 bf16 causal (oracle on batch 0)")
    o, lse, dq, dk, dv = run_fwd_bwd(w, True)
    q, k, v, do = (w.values(n)[:1] for n in ("q", "k", "v", "do"))
    O, L = oracle.ref_fwd(q, k, v, causal=True, scale=w.scale)
    assert_close("O", o[:1], O, TOL_BF16)
    assert_close("LSE", lse[:1], L, TOL_BF16)
    dQ, dK, dV = oracle.ref_bwd(q, k, v, do, causal=True, scale=w.scale)
    assert_close("dQ", dq[:1], dQ, TOL_BF16)
    assert_close("dK", dk[:1], dK, TOL_BF16)
    assert_close("dV", dv[:1], dV, TOL_BF16)


SHAPES = [
    # (B, Hq, Hkv, Nq, Nk, d, causal)
    (1, 1, 1, 1, 1, 64, True),
    (1, 2, 2, 63, 63, 128, True),
    (2, 2, 1, 65, 65, 64, False),
    (1, 4, 2, 257, 257, 128, True),       # GQA g=2, ragged
    (1, 8, 1, 300, 300, 64, True),        # MQA g=8
    (1, 4, 4, 100, 90, 128, False),       # Nq != Nk
    (1, 2, 2, 77, 333, 64, True),         # bottom-right causal
    (2, 4, 1, 1000, 1000, 128, True),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}H{}x{}N{}x{}d{}{}".format(*s[:6], "c" if s[6] else ""))
def test_bwd_edge_shapes(shape, dtype):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    w = W.random_case(sum(shape[:6]) + 3, B, Hq, Hkv, Nq, Nk, d, dtype=dtype, with_do=True)
    announce(f"bwd edge {shape} {dtype}")
    o, lse, dq, dk, dv = run_fwd_bwd(w, causal)
    q, k, v, do = (w.values(n) for n in ("q", "k", "v", "do"))
    dQ, dK, dV = oracle.ref_bwd(q, k, v, do, causal=causal, scale=w.scale)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert_close("dQ", dq, dQ, tol)
    assert_close("dK", dk, dK, tol)
    assert_close("dV", dv, dV, tol)


def test_bf16_gradients():
    """grad_dtype bf16: the float32 result rounded to bf16 (same tolerance)."""
    import torch
    w = W.random_case(41, 1, 4, 2, 512, 512, 128, with_do=True)
    _, _, dq, dk, dv = run_fwd_bwd(w, True, grad_dtype=torch.bfloat16)
    q, k, v, do = (w.values(n) for n in ("q", "k", "v", "do"))
    dQ, dK, dV = oracle.ref_bwd(q, k, v, do, causal=True, scale=w.scale)
    assert_close("dQ(bf16)", dq, dQ, TOL_BF16)
    assert_close("dK(bf16)", dk, dK, TOL_BF16)
    assert_close("dV(bf16)", dv, dV, TOL_BF16)


def test_bwd_is_deterministic():
    w = W.random_case(43, 2, 8, 2, 700, 700, 128, with_do=True)
    a = run_fwd_bwd(w, True)
    b = run_fwd_bwd(w, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_gradient_identities_on_gpu():
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i (MHA), within bf16 tolerance."""
    w = W.random_case(47, 1, 2, 2, 384, 384, 64, with_do=True)
    _, _, dq, dk, dv = run_fwd_bwd(w, True)
    assert np.abs(dk.sum(axis=2)).max() <= 2e-2 * np.sqrt(384)
    assert np.abs(dv.sum(axis=2) - w.values("do").astype(np.float64).sum(axis=2)).max() <= 2e-2 * np.sqrt(384)


def test_backward_beyond_2gib():
    """64 heads of 200000 queries against 64 keys each, d = 128, non-causal: Q,
    dO and O are 3.3 GB and dQ (float32) 6.6 GB, so byte offsets pass 2^31.
    Inputs come from an integer hash of their indices, built on the GPU and
    re-derived on the host; the fp64 oracle (ref_bwd) checks dK and dV of two
    whole heads (the last among them) and dQ on sampled rows of those heads,
    the last rows included.

    Magnitude: each dK and dV element sums 200000 terms, so with dO of the
    hash's size (|x| < 2) the gradients reach ~80 and the absolute bf16 bound
    would be a relative one of 2.5e-4.  dO is therefore the hash times 2^-6
    (exact in bf16; the gradients are linear in dO, so this scales results and
    rounding errors alike by 2^-6), which puts the gradients at the size the
    configurations' N(0,1) inputs give (|grad| up to ~2), and the usual
    absolute bf16 tolerance applies unchanged."""
    import torch
    H, Nq, Nk, d = 64, 200_000, 64, 128
    do_scale = 2.0 ** -6
    announce(f"backward with Q, dO, O of {H * Nq * d * 2 / 2**30:.1f} GiB each")
    dev = "cuda:0"
    cols = torch.arange(d, device=dev, dtype=torch.int64)[None, :]
    rows = torch.arange(Nq, device=dev, dtype=torch.int64)[:, None]
    keys = torch.arange(Nk, device=dev, dtype=torch.int64)[:, None]
    q = torch.empty((1, H, Nq, d), dtype=torch.bfloat16, device=dev)
    do = torch.empty_like(q)
    k = torch.empty((1, H, Nk, d), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    for h in range(H):
        q[0, h] = W.hash_values(rows + h * Nq, cols, 3).to(torch.bfloat16)
        do[0, h] = (W.hash_values(rows + h * Nq, cols, 4) * do_scale).to(torch.bfloat16)
        k[0, h] = W.hash_values(keys + h * Nk, cols, 1).to(torch.bfloat16)
        v[0, h] = W.hash_values(keys + h * Nk, cols, 2).to(torch.bfloat16)
    o, lse = fa.fwd(q, k, v, causal=False)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=False)
    torch.cuda.synchronize()
    colsn = np.arange(d, dtype=np.int64)[None, :]
    for h in (5, H - 1):
        qn = W.hash_values(np.arange(Nq, dtype=np.int64)[:, None] + h * Nq, colsn, 3)
        don = W.hash_values(np.arange(Nq, dtype=np.int64)[:, None] + h * Nq, colsn, 4) * do_scale
        kn = W.hash_values(np.arange(Nk, dtype=np.int64)[:, None] + h * Nk, colsn, 1)
        vn = W.hash_values(np.arange(Nk, dtype=np.int64)[:, None] + h * Nk, colsn, 2)
        dQ, dK, dV = oracle.ref_bwd(qn[None, None], kn[None, None], vn[None, None], don[None, None], causal=False)
        print(f"  head {h}: max |dK| {np.abs(dK).max():.3f}, max |dV| {np.abs(dV).max():.3f}", flush=True)
        assert_close(f"dK[h={h}]", to_host(dk[0, h]), dK[0, 0], TOL_BF16)
        assert_close(f"dV[h={h}]", to_host(dv[0, h]), dV[0, 0], TOL_BF16)
        sel = np.r_[np.random.Generator(np.random.PCG64(h)).integers(0, Nq, 256), np.arange(Nq - 8, Nq)]
        assert_close(f"dQ[h={h}, rows]", to_host(dq[0, h][torch.from_numpy(sel).to(dev)]), dQ[0, 0][sel], TOL_BF16)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_delta_from_stored_o_on_correlated_values(causal):
    """D_i = dO_i . O_i is formed from the stored (bf16) O, so the kernel's D
    differs from the exact one by delta_i = dO_i . (O_i - O_exact,i).  That
    enters the gradients linearly: dQ_i gains -scale delta_i sum_j P_ij k_j
    and dK_j gains -scale sum_i P_ij delta_i q_i (dV does not use D).  With
    values that are nearly equal (v_j = vbar + 2^-5 noise), dP_ij - D_i nearly
    cancels and this term is far above the usual bf16 level; the test checks
    that the kernel's gradients equal the oracle's plus exactly this term, to
    the bf16 tolerance, and that without the term they would not."""
    import torch
    rng = np.random.Generator(np.random.PCG64(77))
    B, H, N, d = 1, 2, 256, 128
    w = W.random_case(79, B, H, H, N, N, d, with_do=True)
    vbar = rng.standard_normal((1, 1, 1, d))
    v = vbar + 2.0 ** -5 * rng.standard_normal((B, H, N, d))
    w.tensors["v"] = W.f32_to_bf16_bits(v.astype(np.float32))
    announce(f"backward, nearly equal values, {'causal' if causal else 'full'}")
    o, lse, dq, dk, dv = run_fwd_bwd(w, causal)
    q, k, vv, do = (w.values(n).astype(np.float64) for n in ("q", "k", "v", "do"))
    scale = 1.0 / np.sqrt(d)
    O, _ = oracle.ref_fwd(q, k, vv, causal=causal)
    P = oracle.ref_probs(q, k, causal=causal)
    dQ, dK, dV = oracle.ref_bwd(q, k, vv, do, causal=causal)
    delta = (do * (o - O)).sum(-1)                                    # [B, H, N]
    dQ_pred = dQ - scale * delta[..., None] * (P @ k)
    dK_pred = dK - scale * np.swapaxes(P, -1, -2) @ (delta[..., None] * q)
    m_plain = oracle.compare(dq, dQ)
    print(f"  dQ without the D term: rel_l2={m_plain['rel_l2']:.3e}", flush=True)
    assert m_plain["rel_l2"] > 5e-3, "inputs do not exercise the D rounding"
    assert_close("dQ (with the D term)", dq, dQ_pred, TOL_BF16)
    assert_close("dK (with the D term)", dk, dK_pred, TOL_BF16)
    assert_close("dV", dv, dV, TOL_BF16)
