"""fa_fwd on the GPU against the fp64 oracle (tolerances: bf16 inputs max-abs
2e-2 and rel-L2 5e-3; fp32 inputs max-abs 1e-5), at the benchmark
configurations and at ragged, grouped and degenerate shapes."""
import numpy as np
import pytest

import exact_io_aware_16_amd as fa
import oracle
import workloads as W
from gpu_helpers import TOL_BF16, TOL_F32, announce, assert_close, to_device, to_host

pytestmark = pytest.mark.gpu


def run_fwd(w, causal):
    q, k, v = (to_device(w.tensors[n]) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal=causal, scale=w.scale)
    return to_host(o), to_host(lse)


def test_config1_single_head_fp32():
    w = W.make_config(1)
    announce("config 1: B1 H1 N256 d64 fp32 non-causal")
    o, lse = run_fwd(w, False)
    O, L = oracle.ref_fwd(w.values("q"), w.values("k"), w.values("v"), causal=False, scale=w.scale)
    assert_close("O", o, O, TOL_F32)
    assert_close("LSE", lse, L, TOL_F32)


def test_config2_causal_bf16_full():
    w = W.make_config(2)
    announce("config 2: B4 H16 N2048 d64 bf16 causal (full oracle)")
    o, lse = run_fwd(w, True)
    O, L = oracle.ref_fwd(w.values("q"), w.values("k"), w.values("v"), causal=True, scale=w.scale)
    assert_close("O", o, O, TOL_BF16)
    assert_close("LSE", lse, L, TOL_BF16)


def test_config3_llama_causal_outliers_sampled_rows():
    w = W.make_config(3)
    announce("config 3: B2 H32 N8192 d128 bf16 causal, 1% K rows x8, 512 sampled rows")
    o, lse = run_fwd(w, True)
    rows = w.sample_rows
    O, L = oracle.ref_fwd_rows(w.values("q"), w.values("k"), w.values("v"), rows, causal=True, scale=w.scale)
    og = np.stack([o[b, h, i] for b, h, i in rows])
    lg = np.array([lse[b, h, i] for b, h, i in rows])
    assert_close("O[rows]", og, O, TOL_BF16)
    assert_close("LSE[rows]", lg, L, TOL_BF16)
    # rows that attend to an outlier key with a large score exercise the rescale
    assert np.isfinite(lse).all()


def test_config5_forward_sampled_rows():
    w = W.make_config(5)
    announce("config 5 forward: B2 H16 N4096 d128 bf16 causal, 512 sampled rows")
    o, lse = run_fwd(w, True)
    rows = W.sampled_query_rows(5, w.B, w.Hq, w.Nq, 512)
    O, L = oracle.ref_fwd_rows(w.values("q"), w.values("k"), w.values("v"), rows, causal=True, scale=w.scale)
    assert_close("O[rows]", np.stack([o[b, h, i] for b, h, i in rows]), O, TOL_BF16)
    assert_close("LSE[rows]", np.array([lse[b, h, i] for b, h, i in rows]), L, TOL_BF16)


@pytest.mark.parametrize("shape", [
    # (B, Hq, Hkv, Nq, Nk, d, causal): grids large enough for two query tiles per wave at d = 64
    (1, 32, 32, 4096, 4096, 64, False),
    (1, 64, 8, 4000, 4000, 64, True),     # GQA g=8, ragged last query block
], ids=lambda s: "B{}H{}x{}N{}x{}d{}{}".format(*s[:6], "c" if s[6] else ""))
def test_d64_large_grids_sampled_rows(shape):
    """The d = 64 kernel takes two 32-query tiles per wave on large grids; 512
    sampled rows against the oracle (the small shapes elsewhere take one)."""
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    w = W.random_case(sum(shape[:6]), B, Hq, Hkv, Nq, Nk, d)
    announce(f"d64 large grid {shape}")
    o, lse = run_fwd(w, causal)
    rows = W.sampled_query_rows(7, B, Hq, Nq, 512)
    O, L = oracle.ref_fwd_rows(w.values("q"), w.values("k"), w.values("v"), rows, causal=causal, scale=w.scale)
    assert_close("O[rows]", np.stack([o[b, h, i] for b, h, i in rows]), O, TOL_BF16)
    assert_close("LSE[rows]", np.array([lse[b, h, i] for b, h, i in rows]), L, TOL_BF16)


SHAPES = [
    # (B, Hq, Hkv, Nq, Nk, d, causal)
    (1, 1, 1, 1, 1, 64, False),
    (1, 2, 2, 1, 1, 128, True),
    (2, 2, 1, 63, 63, 64, True),
    (1, 3, 3, 65, 65, 128, True),
    (1, 2, 2, 257, 257, 64, False),
    (1, 4, 1, 1000, 1000, 128, True),     # MQA, ragged
    (2, 8, 2, 300, 300, 64, True),        # GQA g=4
    (1, 8, 1, 129, 513, 128, False),      # Nq != Nk, MQA g=8
    (1, 4, 4, 100, 90, 64, False),        # the GQA page's Lq/Lk
    (1, 2, 2, 77, 300, 128, True),        # bottom-right causal, Nq < Nk
    (1, 1, 1, 2048, 2048, 64, True),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}H{}x{}N{}x{}d{}{}".format(*s[:6], "c" if s[6] else ""))
def test_edge_shapes(shape, dtype):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    w = W.random_case(sum(shape[:6]), B, Hq, Hkv, Nq, Nk, d, dtype=dtype)
    announce(f"fwd edge {shape} {dtype}")
    o, lse = run_fwd(w, causal)
    O, L = oracle.ref_fwd(w.values("q"), w.values("k"), w.values("v"), causal=causal, scale=w.scale)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert_close("O", o, O, tol)
    assert_close("LSE", lse, L, tol)


def test_arbitrary_scale_and_determinism():
    w = W.random_case(7, 1, 4, 2, 200, 200, 128)
    q, k, v = (to_device(w.tensors[n]) for n in ("q", "k", "v"))
    o1, l1 = fa.fwd(q, k, v, causal=True, scale=0.37)
    o2, l2 = fa.fwd(q, k, v, causal=True, scale=0.37)
    import torch
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    O, L = oracle.ref_fwd(w.values("q"), w.values("k"), w.values("v"), causal=True, scale=0.37)
    assert_close("O", to_host(o1), O, TOL_BF16)
    assert_close("LSE", to_host(l1), L, TOL_BF16)


def test_invalid_arguments_raise():
    import torch
    q = torch.zeros(1, 3, 8, 64, dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(RuntimeError, match="FA_ERR_SHAPE"):
        fa.fwd(q, k, k)
    q = torch.zeros(1, 2, 8, 96, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(RuntimeError, match="FA_ERR_UNSUPPORTED"):
        fa.fwd(q, q, q)


def test_forward_q_and_o_beyond_2gib():
    """MQA with 64 query heads of 200000 rows and 64 keys, d = 128, non-causal:
    Q and O are 3.3 GB each (byte offsets past 2^31), the work small.  Q, K and
    V come from an integer hash of their indices, built on the GPU and
    re-derived on the host for the sampled rows (the last rows of the last head
    among them)."""
    import torch
    Hq, Nq, Nk, d = 64, 200_000, 64, 128
    announce(f"forward with Q and O of {Hq * Nq * d * 2 / 2**30:.1f} GiB each")
    dev = "cuda:0"
    q = torch.empty((1, Hq, Nq, d), dtype=torch.bfloat16, device=dev)
    cols = torch.arange(d, device=dev, dtype=torch.int64)[None, :]
    rows_per_head = torch.arange(Nq, device=dev, dtype=torch.int64)[:, None]
    for h in range(Hq):
        q[0, h] = W.hash_values(rows_per_head + h * Nq, cols, 3).to(torch.bfloat16)
    kj = torch.arange(Nk, device=dev, dtype=torch.int64)[:, None]
    k = W.hash_values(kj, cols, 1).to(torch.bfloat16)[None, None].contiguous()
    v = W.hash_values(kj, cols, 2).to(torch.bfloat16)[None, None].contiguous()
    o, lse = fa.fwd(q, k, v, causal=False)
    rng = np.random.Generator(np.random.PCG64(17))
    heads = np.r_[rng.integers(0, Hq, 500), [Hq - 1] * 12]
    rws = np.r_[rng.integers(0, Nq, 500), np.arange(Nq - 12, Nq)]
    og = o[0, torch.from_numpy(heads).to(dev), torch.from_numpy(rws).to(dev)].float().cpu().numpy().astype(np.float64)
    lg = lse[0, torch.from_numpy(heads).to(dev), torch.from_numpy(rws).to(dev)].cpu().numpy().astype(np.float64)
    del q, o
    torch.cuda.empty_cache()
    colsn = np.arange(d, dtype=np.int64)[None, :]
    kn = W.hash_values(np.arange(Nk, dtype=np.int64)[:, None], colsn, 1)
    vn = W.hash_values(np.arange(Nk, dtype=np.int64)[:, None], colsn, 2)
    qn = W.hash_values((rws + heads * Nq).astype(np.int64)[:, None], colsn, 3)
    # the oracle on the sampled rows: non-causal against one K/V head, so each
    # sampled row is a query head of its own against the same 64 keys
    O, L = oracle.ref_fwd(qn[None, :, None, :], kn[None, None], vn[None, None], causal=False)
    O, L = O[0, :, 0], L[0, :, 0]
    assert_close("O[rows]", og, O, TOL_BF16)
    assert_close("LSE[rows]", lg, L, TOL_BF16)
