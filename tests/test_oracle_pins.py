"""Pins for the CPU oracle: facts fixed by the pages and by the mathematics.

Every check is written against the *definition* (softmax(scale Q K^T) V with a
mask) through a route other than the oracle's own code: the printed
tiled-vs-standard result of handsonai.io DL101 ch. 9 section 3.3, closed forms,
invariants, pure-Python brute force, finite differences, and PyTorch's fp64 CPU
scaled_dot_product_attention + autograd as a library special case.

The checks take the implementation under test as an argument, so
``test_oracle_mutations.py`` can show that a planted mistake fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W
from workloads import random_case, random_lengths

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, *shape):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


# ---------------------------------------------------------------------------
# brute force: pure Python loops over the definition (tiny inputs only)
# ---------------------------------------------------------------------------

def brute_attention(q, k, v, causal, scale, kv_lens=None):
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    O = [[[[0.0] * d for _ in range(Nq)] for _ in range(Hq)] for _ in range(B)]
    L = [[[-math.inf] * Nq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            for i in range(Nq):
                keys = [j for j in range(Nk)
                        if (kv_lens is None or j < kv_lens[b]) and (not causal or j <= i + Nk - Nq)]
                if not keys:
                    continue
                s = {j: scale * sum(float(q[b, h, i, c]) * float(k[b, kh, j, c]) for c in range(d)) for j in keys}
                mx = max(s.values())
                den = sum(math.exp(s[j] - mx) for j in keys)
                for c in range(d):
                    O[b][h][i][c] = sum(math.exp(s[j] - mx) / den * float(v[b, kh, j, c]) for j in keys)
                L[b][h][i] = mx + math.log(den)
    return np.array(O), np.array(L)


# ---------------------------------------------------------------------------
# forward checks, parameterised by fwd(q, k, v, causal, scale, kv_lens) -> (O, LSE)
# ---------------------------------------------------------------------------

def check_brute_force(fwd):
    ok = True
    for seed, (B, Hq, Hkv, Nq, Nk, d, causal) in enumerate([
        (1, 2, 1, 4, 6, 3, True), (2, 2, 2, 5, 5, 2, False), (1, 4, 2, 3, 5, 3, True),
        (1, 1, 1, 6, 4, 2, False)]):
        q, k, v = _rand(seed, B, Hq, Nq, d), _rand(seed + 50, B, Hkv, Nk, d), _rand(seed + 99, B, Hkv, Nk, d)
        sc = 0.7
        O, L = fwd(q, k, v, causal, sc, None)
        Ob, Lb = brute_attention(q, k, v, causal, sc)
        ok &= np.allclose(O, Ob, atol=1e-12, rtol=0) and np.allclose(L, Lb, atol=1e-12, rtol=0)
    # with cache lengths (decode semantics)
    q, k, v = _rand(7, 3, 4, 1, 3), _rand(8, 3, 2, 7, 3), _rand(9, 3, 2, 7, 3)
    lens = [7, 1, 4]
    O, L = fwd(q, k, v, False, 0.5, np.array(lens))
    Ob, Lb = brute_attention(q, k, v, False, 0.5, lens)
    ok &= np.allclose(O, Ob, atol=1e-12, rtol=0) and np.allclose(L, Lb, atol=1e-12, rtol=0)
    return bool(ok)


def check_closed_forms(fwd):
    ok = True
    d = 4
    sc = 1 / math.sqrt(d)
    # N = 1: O = V_0, LSE = scale q.k_0
    q, k, v = _rand(1, 1, 1, 1, d), _rand(2, 1, 1, 1, d), _rand(3, 1, 1, 1, d)
    O, L = fwd(q, k, v, False, sc, None)
    ok &= np.allclose(O[0, 0, 0], v[0, 0, 0], atol=1e-14) and abs(L[0, 0, 0] - sc * q[0, 0, 0] @ k[0, 0, 0]) < 1e-14
    # causal row 0 sees only key 0
    q, k, v = _rand(4, 1, 1, 5, d), _rand(5, 1, 1, 5, d), _rand(6, 1, 1, 5, d)
    O, L = fwd(q, k, v, True, sc, None)
    ok &= np.allclose(O[0, 0, 0], v[0, 0, 0], atol=1e-14) and abs(L[0, 0, 0] - sc * q[0, 0, 0] @ k[0, 0, 0]) < 1e-14
    # N = 2: O = sigmoid(s0 - s1) V0 + sigmoid(s1 - s0) V1, LSE = log(e^s0 + e^s1)
    q, k, v = _rand(7, 1, 1, 1, d), _rand(8, 1, 1, 2, d), _rand(9, 1, 1, 2, d)
    O, L = fwd(q, k, v, False, sc, None)
    s0, s1 = sc * q[0, 0, 0] @ k[0, 0, 0], sc * q[0, 0, 0] @ k[0, 0, 1]
    sig = lambda x: 1 / (1 + math.exp(-x))
    ok &= np.allclose(O[0, 0, 0], sig(s0 - s1) * v[0, 0, 0] + sig(s1 - s0) * v[0, 0, 1], atol=1e-14)
    ok &= abs(L[0, 0, 0] - math.log(math.exp(s0) + math.exp(s1))) < 1e-13
    # Q = 0: uniform weights -> mean of the valid V rows; LSE = ln(count)
    N = 6
    q = np.zeros((1, 1, N, d)); k, v = _rand(10, 1, 1, N, d), _rand(11, 1, 1, N, d)
    O, L = fwd(q, k, v, True, sc, None)
    for i in range(N):
        ok &= np.allclose(O[0, 0, i], v[0, 0, :i + 1].mean(axis=0), atol=1e-14)
        ok &= abs(L[0, 0, i] - math.log(i + 1)) < 1e-14
    # all keys equal: uniform weights for any query
    q = _rand(12, 1, 1, 3, d); k = np.repeat(_rand(13, 1, 1, 1, d), N, axis=2); v = _rand(14, 1, 1, N, d)
    O, _ = fwd(q, k, v, False, sc, None)
    ok &= np.allclose(O[0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (3, d)), atol=1e-14)
    return bool(ok)


def check_rows_sum_to_one():
    P = oracle.ref_probs(_rand(1, 2, 4, 9, 5), _rand(2, 2, 2, 11, 5), causal=True)
    Pn = oracle.ref_probs(_rand(3, 1, 2, 7, 5), _rand(4, 1, 2, 7, 5), causal=False, kv_lens=np.array([3]))
    return bool(np.allclose(P.sum(-1), 1, atol=1e-14) and np.allclose(Pn.sum(-1), 1, atol=1e-14)
                and (P >= 0).all() and np.all(Pn[..., 3:] == 0))


def check_chunked_equals_one_shot(fwd):
    """[TILE]: the block recurrence gives the one-shot result, for any blocking."""
    ok = True
    for causal, Nq, Nk in [(False, 37, 53), (True, 41, 41), (True, 19, 50)]:
        d = 8
        q, k, v = _rand(Nq, 1, 1, Nq, d), _rand(Nk, 1, 1, Nk, d), _rand(Nk + 1, 1, 1, Nk, d)
        O, L = fwd(q, k, v, causal, 0.35, None)
        for bq, bk in [(1, 1), (7, 5), (16, 16), (64, 64), (Nq, 3)]:
            Ot, Lt = oracle.tiled_fwd(q[0, 0], k[0, 0], v[0, 0], bq, bk, causal=causal, scale=0.35)
            ok &= np.abs(Ot - O[0, 0]).max() <= 1e-12 and np.abs(Lt - L[0, 0]).max() <= 1e-12
    return bool(ok)


def check_invariants(fwd):
    ok = True
    d, N = 6, 13
    sc = 0.41
    q, k, v = _rand(21, 2, 4, N, d), _rand(22, 2, 2, N, d), _rand(23, 2, 2, N, d)
    O, L = fwd(q, k, v, True, sc, None)
    # constant V -> constant O
    vc = np.broadcast_to(_rand(24, 1, 1, 1, d), v.shape).copy()
    Oc, _ = fwd(q, k, vc, True, sc, None)
    ok &= np.allclose(Oc, np.broadcast_to(vc[:, :1, :1], Oc.shape), atol=1e-14)
    # V -> alpha V
    Oa, La = fwd(q, k, 3.5 * v, True, sc, None)
    ok &= np.allclose(Oa, 3.5 * O, atol=1e-13) and np.allclose(La, L, atol=0)
    # shifting every key by u leaves O, and shifts LSE_i by scale q_i . u
    u = _rand(25, d)
    Os, Ls = fwd(q, k + u, v, True, sc, None)
    ok &= np.allclose(Os, O, atol=1e-12) and np.allclose(Ls, L + sc * (q @ u), atol=1e-12)
    # GQA equals MHA with repeated K/V heads ([GQA])
    Or, Lr = fwd(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), True, sc, None)
    ok &= np.array_equal(Or, O) and np.array_equal(Lr, L)
    # masked keys get zero weight: change masked K/V, O of earlier rows unchanged bit for bit
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 9:] = 1e3 * _rand(26, 2, 2, N - 9, d)
    v2[:, :, 9:] = 1e30
    O2, L2 = fwd(q, k2, v2, True, sc, None)
    ok &= np.array_equal(O2[:, :, :9], O[:, :, :9]) and np.array_equal(L2[:, :, :9], L[:, :, :9])
    # cache lengths: keys at or beyond len_b never matter
    lens = np.array([5, 13])
    Ol, Ll = fwd(q, k, v, False, sc, lens)
    k3, v3 = k.copy(), v.copy()
    k3[0, :, 5:] = np.inf
    v3[0, :, 5:] = np.nan
    Ol2, Ll2 = fwd(q, k3, v3, False, sc, lens)
    ok &= np.array_equal(Ol, Ol2) and np.array_equal(Ll, Ll2)
    # a row with no valid key: O = 0, LSE = -inf (reading of the pages' silence)
    Oe, Le = fwd(q[:1, :, :2], k[:1], v[:1], False, sc, np.array([0]))
    ok &= np.all(Oe == 0) and np.all(np.isneginf(Le))
    return bool(ok)


def check_torch_sdpa(fwd):
    """Library special case: PyTorch's CPU scaled_dot_product_attention in float64."""
    import torch
    import torch.nn.functional as F
    ok = True
    for seed, (B, Hq, Hkv, Nq, Nk, d, causal) in enumerate([
        (2, 4, 4, 33, 33, 16, True), (1, 8, 2, 20, 29, 8, False), (2, 6, 3, 17, 17, 8, True),
        (1, 4, 1, 12, 30, 8, True)]):
        q, k, v = _rand(seed, B, Hq, Nq, d), _rand(seed + 10, B, Hkv, Nk, d), _rand(seed + 20, B, Hkv, Nk, d)
        O, _ = fwd(q, k, v, causal, 1 / math.sqrt(d), None)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        g = Hq // Hkv
        tk, tv = tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1)
        mask = None
        if causal:
            i = torch.arange(Nq)[:, None]
            j = torch.arange(Nk)[None, :]
            mask = j <= i + (Nk - Nq)
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask).numpy()
        ok &= np.abs(O - ref).max() <= 1e-12
    return bool(ok)


def fwd_oracle(q, k, v, causal, scale, kv_lens):
    return oracle.ref_fwd(q, k, v, causal=causal, scale=scale, kv_lens=kv_lens)


# ---------------------------------------------------------------------------
# the tests
# ---------------------------------------------------------------------------

def test_brute_force():
    assert check_brute_force(fwd_oracle)


def test_closed_forms():
    assert check_closed_forms(fwd_oracle)


def test_rows_of_p_sum_to_one():
    assert check_rows_sum_to_one()


def test_chunked_online_softmax_equals_one_shot():
    assert check_chunked_equals_one_shot(fwd_oracle)


def test_invariants():
    assert check_invariants(fwd_oracle)


def test_matches_torch_sdpa_fp64():
    assert check_torch_sdpa(fwd_oracle)


def test_online_softmax_stats_closed_form():
    """[OS]: the running (m, d) pair equals (max x, sum exp(x - max x)) for any chunking."""
    x = _rand(3, 101) * 5
    m_ref = x.max()
    d_ref = np.exp(x - m_ref).sum()
    for cuts in ([101], [1] * 101, [10, 0, 41, 50], [100, 1]):
        chunks, s = [], 0
        for c in cuts:
            chunks.append(x[s:s + c]); s += c
        m, dn = oracle.online_softmax_stats(chunks)
        assert m == m_ref and abs(dn - d_ref) <= 1e-12 * d_ref


def test_tiled_vs_standard_printed_mse():
    """handsonai.io DL101 ch.9 sec 3.3 prints MSE 0.0000000000 (fp32, Lq 1280, Lk 1152, d 512, 64x64 blocks)."""
    g = json.load(open(os.path.join(GOLD, "tiled_vs_standard.json")))
    Lq, Lk, d, bq, bk = g["Lq"], g["Lk"], g["d"], g["block_q"], g["block_k"]
    rng = np.random.Generator(np.random.PCG64(42))
    Q = rng.standard_normal((Lq, d), dtype=np.float32)
    K = rng.standard_normal((Lk, d), dtype=np.float32)
    V = rng.standard_normal((Lk, d), dtype=np.float32)
    O_ref, L_ref = oracle.ref_fwd(Q[None, None], K[None, None], V[None, None])
    O32, _ = oracle.tiled_fwd(Q, K, V, bq, bk, dtype=np.float32)
    mse = float(np.mean((O32.astype(np.float64) - O_ref[0, 0]) ** 2))
    assert mse < g["mse_upper_bound"], mse
    assert f"{mse:.10f}" == g["printed_mse"]
    O64, L64 = oracle.tiled_fwd(Q, K, V, bq, bk, dtype=np.float64)
    assert np.abs(O64 - O_ref[0, 0]).max() <= 1e-12
    assert np.abs(L64 - L_ref[0, 0]).max() <= 1e-12


def test_gqa_output_shapes_printed():
    """DL101 ch.9 sec 3.1/3.2 print the output shape [32, 8, 100, 64] for MQA and GQA."""
    g = json.load(open(os.path.join(GOLD, "gqa_shapes.json")))
    for c in g["cases"]:
        # shrink batch for speed; the printed shape's batch is checked by arithmetic
        B = 2
        q = _rand(1, B, c["n_heads"], c["Lq"], c["d_head"])
        k = _rand(2, B, c["n_groups"], c["Lk"], c["d_head"])
        v = _rand(3, B, c["n_groups"], c["Lk"], c["d_head"])
        O, L = oracle.ref_fwd(q, k, v)
        assert list(O.shape) == [B] + c["printed_output_shape"][1:]
        assert L.shape == (B, c["n_heads"], c["Lq"])
        # and it equals MHA with each K/V head repeated for its group
        rep = c["n_heads"] // c["n_groups"]
        O2, _ = oracle.ref_fwd(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1))
        assert np.array_equal(O, O2)


def test_rows_variant_matches_full():
    w = random_case(3, 2, 4, 2, 40, 40, 16, dtype="f32")
    q, k, v = w.values("q"), w.values("k"), w.values("v")
    for causal in (False, True):
        O, L = oracle.ref_fwd(q, k, v, causal=causal)
        rows = np.array([[0, 0, 0], [1, 3, 39], [0, 2, 17], [1, 1, 5]])
        Or, Lr = oracle.ref_fwd_rows(q, k, v, rows, causal=causal)
        for r, (b, h, i) in enumerate(rows):
            assert np.abs(Or[r] - O[b, h, i]).max() <= 1e-12
            assert abs(Lr[r] - L[b, h, i]) <= 1e-12


# ---------------------------------------------------------------------------
# ref_fwd_rows: the definition one query row at a time (sampled-row parity of
# the large workloads), checked against pure-Python brute force on causal
# shapes with Nq < Nk (bottom-right offset Nk - Nq > 0) and grouped heads
# ---------------------------------------------------------------------------

def check_rows_variant(rows_fn):
    """rows_fn(q, k, v, rows, causal, scale) -> (O [R, d], LSE [R])."""
    ok = True
    for seed, (B, Hq, Hkv, Nq, Nk, d, causal) in enumerate([
            (2, 4, 2, 3, 7, 3, True),     # offset 4, two query heads per K/V head
            (1, 6, 3, 5, 5, 2, True),     # Nq == Nk
            (1, 4, 1, 2, 9, 3, True),     # offset 7, one K/V head for all
            (2, 4, 2, 4, 6, 2, False)]):
        q = _rand(seed + 300, B, Hq, Nq, d)
        k, v = _rand(seed + 310, B, Hkv, Nk, d), _rand(seed + 320, B, Hkv, Nk, d)
        Ob, Lb = brute_attention(q, k, v, causal, 0.6)
        rows = np.array([[b, h, i] for b in range(B) for h in range(Hq) for i in range(Nq)])
        Or, Lr = rows_fn(q, k, v, rows, causal, 0.6)
        for r, (b, h, i) in enumerate(rows):
            ok &= np.abs(Or[r] - Ob[b, h, i]).max() <= 1e-12 and abs(Lr[r] - Lb[b, h, i]) <= 1e-12
    return bool(ok)


def rows_oracle(q, k, v, rows, causal, scale):
    return oracle.ref_fwd_rows(q, k, v, rows, causal=causal, scale=scale)


def test_rows_variant_brute_force_offset_and_groups():
    assert check_rows_variant(rows_oracle)


def test_rows_variant_matches_full_bottom_right_gqa():
    """Nq < Nk causal with grouped heads: every sampled row equals ref_fwd's."""
    w = random_case(4, 2, 8, 2, 24, 61, 16, dtype="f32")
    q, k, v = w.values("q"), w.values("k"), w.values("v")
    O, L = oracle.ref_fwd(q, k, v, causal=True)
    rows = np.array([[b, h, i] for b in range(2) for h in (0, 3, 4, 7) for i in (0, 1, 11, 23)])
    Or, Lr = oracle.ref_fwd_rows(q, k, v, rows, causal=True)
    for r, (b, h, i) in enumerate(rows):
        assert np.abs(Or[r] - O[b, h, i]).max() <= 1e-12
        assert abs(Lr[r] - L[b, h, i]) <= 1e-12


# ---------------------------------------------------------------------------
# compare: the metric behind every parity test
# ---------------------------------------------------------------------------

def _brute_metrics(g, r):
    """max |g - r| and ||g - r|| / ||r|| by plain Python loops over finite r."""
    mx, num, den = 0.0, 0.0, 0.0
    for a, b in zip(np.ravel(g).tolist(), np.ravel(r).tolist()):
        if math.isfinite(b):
            mx = max(mx, abs(a - b))
            num += (a - b) ** 2
            den += b * b
    return mx, math.sqrt(num) / math.sqrt(den)


def check_compare(cmp):
    ok = True
    mism = lambda m: bool(m.get("nonfinite_mismatch"))
    # hand-built: ref norm 5, difference (0, 0.5)
    m = cmp(np.array([3.0, 4.5]), np.array([3.0, 4.0]))
    ok &= m["max_abs"] == 0.5 and abs(m["rel_l2"] - 0.1) < 1e-15 and not mism(m)
    # the largest deviation is negative; difference norm 0.5, ref norm 10
    r = np.ones(100)
    g = r.copy()
    g[3] += 0.3
    g[70] -= 0.4
    m = cmp(g, r)
    ok &= abs(m["max_abs"] - 0.4) < 1e-15 and abs(m["rel_l2"] - 0.05) < 1e-15
    # relative to the reference's norm, not the result's (g = 2r: rel-L2 = 1)
    m = cmp(np.array([6.0, 8.0]), np.array([3.0, 4.0]))
    ok &= m["max_abs"] == 4.0 and abs(m["rel_l2"] - 1.0) < 1e-15
    # equal arrays, any shape
    r = _rand(5, 3, 4, 5)
    m = cmp(r.copy(), r)
    ok &= m["max_abs"] == 0.0 and m["rel_l2"] == 0.0
    # brute force on random 3-d arrays
    g = r + 1e-3 * _rand(6, 3, 4, 5)
    mx, rel = _brute_metrics(g, r)
    m = cmp(g, r)
    ok &= abs(m["max_abs"] - mx) < 1e-15 and abs(m["rel_l2"] - rel) < 1e-13
    # -inf in the same places (rows without keys) is equal and left out of the norms
    m = cmp(np.array([-np.inf, 2.5, -np.inf]), np.array([-np.inf, 2.0, -np.inf]))
    ok &= m["max_abs"] == 0.5 and m["rel_l2"] == 0.25 and not mism(m)
    # a whole row of -inf on both sides
    m = cmp(np.full(4, -np.inf), np.full(4, -np.inf))
    ok &= m["max_abs"] == 0.0 and m["rel_l2"] == 0.0 and not mism(m)
    # non-finite patterns that differ, either way, and +inf for -inf
    for g2, r2 in ([0.0, 1.0], [-np.inf, 1.0]), ([-np.inf, 1.0], [0.0, 1.0]), ([np.inf, 1.0], [-np.inf, 1.0]):
        m = cmp(np.array(g2), np.array(r2))
        ok &= mism(m) and m["max_abs"] == np.inf and m["rel_l2"] == np.inf
    # NaN in the result fails, also where the reference is -inf
    for g2, r2 in ([np.nan, 1.0], [0.0, 1.0]), ([np.nan, 1.0], [-np.inf, 1.0]):
        ok &= mism(cmp(np.array(g2), np.array(r2)))
    # an all-zero reference: rel-L2 is the absolute norm of the difference
    m = cmp(np.array([0.0, 3e-3, 4e-3]), np.zeros(3))
    ok &= m["max_abs"] == 4e-3 and abs(m["rel_l2"] - 5e-3) < 1e-15
    # arrays of different shapes are an error, not a silent broadcast
    try:
        cmp(np.zeros((2, 3)), np.zeros(3))
        ok = False
    except ValueError:
        pass
    return bool(ok)


def test_compare_metrics():
    assert check_compare(oracle.compare)


def test_decode_equals_forward_prefix():
    w = random_case(5, 3, 8, 2, 1, 50, 16, dtype="f32")
    q, k, v = w.values("q"), w.values("k"), w.values("v")
    lens = random_lengths(1, 3, 1, 50)
    O, L = oracle.ref_decode(q, k, v, lens)
    for b in range(3):
        n = int(lens[b])
        Of, Lf = oracle.ref_fwd(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n])
        assert np.abs(O[b] - Of[0]).max() <= 1e-13
        assert np.abs(L[b] - Lf[0, :, 0]).max() <= 1e-13
    # brute force on the same problem
    Ob, Lb = brute_attention(q[:, :, :, :4], k[:, :, :, :4], v[:, :, :, :4], False, 0.25, list(lens))
    Oo, Lo = oracle.ref_decode(q[:, :, :, :4], k[:, :, :, :4], v[:, :, :, :4], lens, scale=0.25)
    assert np.abs(Oo - Ob).max() <= 1e-12 and np.abs(Lo - Lb[:, :, 0]).max() <= 1e-12


def test_split_merge_equals_unsplit():
    q, k, v = _rand(1, 1, 2, 3, 8), _rand(2, 1, 2, 100, 8), _rand(3, 1, 2, 100, 8)
    O, L = oracle.ref_fwd(q, k, v)
    for cuts in ([0, 100], [0, 10, 55, 100], [0, 1, 2, 3, 99, 100], [0, 30, 30, 100]):
        parts_o, parts_l = [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            if b > a:
                Oi, Li = oracle.ref_fwd(q, k[:, :, a:b], v[:, :, a:b])
            else:
                Oi, Li = np.zeros_like(O), np.full_like(L, -np.inf)
            parts_o.append(Oi); parts_l.append(Li)
        Om, Lm = oracle.merge_partials(np.stack(parts_o), np.stack(parts_l))
        assert np.abs(Om - O).max() <= 1e-13 and np.abs(Lm - L).max() <= 1e-13
    # all parts empty -> O = 0, LSE = -inf
    Om, Lm = oracle.merge_partials(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf))
    assert np.all(Om == 0) and np.all(np.isneginf(Lm))


# ---------------------------------------------------------------------------
# backward checks, parameterised by bwd(q, k, v, do, causal, scale) -> (dQ, dK, dV)
# ---------------------------------------------------------------------------

def _loss(q, k, v, do, causal, scale):
    O, _ = oracle.ref_fwd(q, k, v, causal=causal, scale=scale)
    return float((O * do).sum())


def check_finite_differences(bwd):
    ok = True
    for seed, (B, Hq, Hkv, Nq, Nk, d, causal) in enumerate([
        (1, 2, 1, 5, 5, 3, True), (1, 2, 2, 4, 6, 3, False), (2, 2, 1, 3, 5, 2, True)]):
        q, k, v = _rand(seed, B, Hq, Nq, d), _rand(seed + 5, B, Hkv, Nk, d), _rand(seed + 9, B, Hkv, Nk, d)
        do = _rand(seed + 13, B, Hq, Nq, d)
        sc = 0.6
        grads = bwd(q, k, v, do, causal, sc)
        eps = 1e-6
        for gi, x in enumerate((q, k, v)):
            num = np.zeros_like(x)
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                xp = x.copy(); xp[idx] += eps
                xm = x.copy(); xm[idx] -= eps
                args_p = [q, k, v]; args_p[gi] = xp
                args_m = [q, k, v]; args_m[gi] = xm
                num[idx] = (_loss(*args_p, do, causal, sc) - _loss(*args_m, do, causal, sc)) / (2 * eps)
            ok &= np.abs(num - grads[gi]).max() <= 1e-7 * max(1.0, np.abs(num).max())
    return bool(ok)


def check_gradient_identities(bwd):
    ok = True
    B, H, N, d = 2, 3, 17, 5
    q, k, v, do = _rand(1, B, H, N, d), _rand(2, B, H, N, d), _rand(3, B, H, N, d), _rand(4, B, H, N, d)
    for causal in (False, True):
        dQ, dK, dV = bwd(q, k, v, do, causal, 0.45)
        # each row of dS sums to zero -> sum_j dK_j = 0
        ok &= np.abs(dK.sum(axis=2)).max() <= 1e-12
        # rows of P sum to one -> sum_j dV_j = sum_i dO_i
        ok &= np.abs(dV.sum(axis=2) - do.sum(axis=2)).max() <= 1e-12
        # linearity in dO
        dQ2, dK2, dV2 = bwd(q, k, v, 2.0 * do + do[:, :, ::-1], causal, 0.45)
        dQ3, dK3, dV3 = bwd(q, k, v, do[:, :, ::-1], causal, 0.45)
        ok &= np.allclose(dQ2, 2 * dQ + dQ3, atol=1e-12) and np.allclose(dV2, 2 * dV + dV3, atol=1e-12)
        ok &= np.allclose(dK2, 2 * dK + dK3, atol=1e-12)
    return bool(ok)


def check_torch_autograd(bwd):
    import torch
    import torch.nn.functional as F
    ok = True
    for seed, (B, Hq, Hkv, N, d, causal) in enumerate([(2, 4, 2, 19, 8, True), (1, 2, 2, 23, 16, False)]):
        q, k, v, do = (_rand(seed + s, *shp) for s, shp in enumerate(
            [(B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d), (B, Hq, N, d)]))
        dQ, dK, dV = bwd(q, k, v, do, causal, 1 / math.sqrt(d))
        tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
        g = Hq // Hkv
        out = F.scaled_dot_product_attention(tq, tk.repeat_interleave(g, 1), tv.repeat_interleave(g, 1),
                                             is_causal=causal)
        out.backward(torch.from_numpy(do))
        ok &= np.abs(tq.grad.numpy() - dQ).max() <= 1e-12
        ok &= np.abs(tk.grad.numpy() - dK).max() <= 1e-12
        ok &= np.abs(tv.grad.numpy() - dV).max() <= 1e-12
    return bool(ok)


def bwd_oracle(q, k, v, do, causal, scale):
    return oracle.ref_bwd(q, k, v, do, causal=causal, scale=scale)


def test_bwd_finite_differences():
    assert check_finite_differences(bwd_oracle)


def test_bwd_gradient_identities():
    assert check_gradient_identities(bwd_oracle)


def test_bwd_matches_torch_autograd_fp64():
    assert check_torch_autograd(bwd_oracle)


def test_bwd_delta_identity():
    """D_i = sum_j P_ij dP_ij equals dO_i . O_i (the identity the GPU backward uses)."""
    q, k, v, do = _rand(1, 1, 2, 9, 4), _rand(2, 1, 2, 9, 4), _rand(3, 1, 2, 9, 4), _rand(4, 1, 2, 9, 4)
    P = oracle.ref_probs(q, k, causal=True)
    O, _ = oracle.ref_fwd(q, k, v, causal=True)
    dP = np.einsum("bhid,bhjd->bhij", do, v)
    D1 = (P * dP).sum(-1)
    D2 = (do * O).sum(-1)
    assert np.abs(D1 - D2).max() <= 1e-13


# ---------------------------------------------------------------------------
# chunk decode (Nq new tokens against the cache; DL101 chapter 9, sections 1.1
# and 1.2), checks parameterised by chunk(q, k, v, lens, causal, scale)
# ---------------------------------------------------------------------------

def check_chunk_brute_force(chunk):
    """Per sequence: the pure-Python definition over its own len_b keys, causal
    bottom-right aligned to len_b (token t sees keys j <= t + len_b - Nq)."""
    ok = True
    for seed, (B, Hq, Hkv, Nq, Nmax, d, lens) in enumerate([
            (3, 4, 2, 3, 7, 3, [7, 5, 2]), (2, 2, 1, 4, 6, 2, [4, 0]), (1, 6, 3, 2, 5, 4, [1])]):
        q, k, v = _rand(seed + 300, B, Hq, Nq, d), _rand(seed + 310, B, Hkv, Nmax, d), _rand(seed + 320, B, Hkv, Nmax, d)
        for causal in (True, False):
            O, L = chunk(q, k, v, np.array(lens), causal, 0.6)
            for b in range(B):
                n = lens[b]
                Ob, Lb = brute_attention(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], causal, 0.6)
                ok &= np.allclose(O[b], Ob[0], atol=1e-12, rtol=0) and np.allclose(L[b], Lb[0], atol=1e-12, rtol=0)
    return bool(ok)


def check_chunk_rows_are_decodes(chunk):
    """Token t of a causal chunk is a one-token decode with the cache cut to
    len_b - (Nq - 1 - t) keys; without causal, with all len_b keys."""
    B, Hq, Hkv, Nq, Nmax, d = 3, 8, 2, 5, 40, 8
    q, k, v = _rand(401, B, Hq, Nq, d), _rand(402, B, Hkv, Nmax, d), _rand(403, B, Hkv, Nmax, d)
    lens = np.array([40, 17, 3])
    Oc, Lc = chunk(q, k, v, lens, True, 0.3)
    On, Ln = chunk(q, k, v, lens, False, 0.3)
    ok = True
    for t in range(Nq):
        cut = np.maximum(lens - (Nq - 1 - t), 0)
        Od, Ld = oracle.ref_decode(q[:, :, t:t + 1], k, v, cut, scale=0.3)
        fin = np.isfinite(Ld)
        ok &= np.abs(Oc[:, :, t] - Od[:, :, 0]).max() <= 1e-13 and np.array_equal(np.isneginf(Lc[:, :, t]), ~fin)
        ok &= np.abs(Lc[:, :, t][fin] - Ld[fin]).max() <= 1e-13
        Od, Ld = oracle.ref_decode(q[:, :, t:t + 1], k, v, lens, scale=0.3)
        ok &= np.abs(On[:, :, t] - Od[:, :, 0]).max() <= 1e-13 and np.abs(Ln[:, :, t] - Ld).max() <= 1e-13
    return bool(ok)


def check_chunk_special_cases(chunk):
    """Nq = 1 is decode; a chunk longer than its sequence leaves the first
    tokens without keys (O = 0, LSE = -inf); keys past len_b never matter."""
    ok = True
    q, k, v = _rand(501, 2, 4, 1, 8), _rand(502, 2, 2, 30, 8), _rand(503, 2, 2, 30, 8)
    lens = np.array([30, 9])
    O, L = chunk(q, k, v, lens, True, 0.4)
    Od, Ld = oracle.ref_decode(q, k, v, lens, scale=0.4)
    ok &= np.abs(O - Od).max() <= 1e-14 and np.abs(L[:, :, 0] - Ld).max() <= 1e-14
    q = _rand(504, 2, 4, 6, 8)
    lens = np.array([4, 30])
    O, L = chunk(q, k, v, lens, True, 0.4)
    ok &= np.all(O[0, :, :2] == 0) and np.all(np.isneginf(L[0, :, :2])) and np.all(np.isfinite(L[0, :, 2:]))
    # token 2 of sequence 0 sees exactly key 0: O = V_0, LSE = scale q.k_0
    ok &= np.allclose(O[0, :, 2], np.repeat(v[0, :, 0], 2, axis=0), atol=1e-14)
    ok &= np.allclose(L[0, :, 2], 0.4 * np.einsum("hd,hd->h", q[0, :, 2], np.repeat(k[0, :, 0], 2, axis=0)), atol=1e-13)
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 4:] = np.inf
    v2[0, :, 4:] = np.nan
    O2, L2 = chunk(q, k2, v2, lens, True, 0.4)
    ok &= np.array_equal(O2, O) and np.array_equal(L2, L)
    return bool(ok)


def chunk_oracle(q, k, v, lens, causal, scale):
    return oracle.ref_decode_chunk(q, k, v, lens, causal=causal, scale=scale)


def test_decode_chunk_brute_force():
    assert check_chunk_brute_force(chunk_oracle)


def test_decode_chunk_rows_are_decodes():
    assert check_chunk_rows_are_decodes(chunk_oracle)


def test_decode_chunk_special_cases():
    assert check_chunk_special_cases(chunk_oracle)


# ---------------------------------------------------------------------------
# paged cache (unite.ai "What is FlashAttention", sources section, naming
# vLLM's PagedAttention), checks parameterised by
# paged(q, k_pages, v_pages, table, lens, page_size, causal, scale)
# ---------------------------------------------------------------------------

def _pool_from_contiguous(k, page_size):
    """[B, Hkv, max_pages*P, d] -> pool [B*max_pages, Hkv, P, d] with sequence b's
    page p at physical index b*max_pages + p (a plain reshape)."""
    B, Hkv, N, d = k.shape
    mp = N // page_size
    return k.reshape(B, Hkv, mp, page_size, d).transpose(0, 2, 1, 3, 4).reshape(B * mp, Hkv, page_size, d)


def check_paged_contiguous_case(paged):
    """An identity block table over a reshaped contiguous cache is the chunk
    decode of that cache (a case that reduces to the pinned chunk oracle)."""
    ok = True
    for seed, (B, Hq, Hkv, Nq, P, mp, d, lens) in enumerate([
            (3, 8, 2, 1, 32, 4, 8, [128, 70, 0]), (2, 4, 1, 3, 16, 5, 4, [80, 2])]):
        q = _rand(seed + 600, B, Hq, Nq, d)
        k, v = _rand(seed + 610, B, Hkv, mp * P, d), _rand(seed + 620, B, Hkv, mp * P, d)
        table = np.arange(B * mp).reshape(B, mp)
        for causal in (True, False):
            O, L = paged(q, _pool_from_contiguous(k, P), _pool_from_contiguous(v, P), table, np.array(lens), P,
                         causal, 0.45)
            Oc, Lc = oracle.ref_decode_chunk(q, k, v, np.array(lens), causal=causal, scale=0.45)
            ok &= np.array_equal(O, Oc) and np.array_equal(L, Lc)
    return bool(ok)


def check_paged_brute_force(paged):
    """Pure Python: key j of sequence b is row j % P of page table[b][j // P]."""
    B, Hq, Hkv, Nq, P, npages, mp, d = 2, 4, 2, 2, 4, 7, 3, 3
    q = _rand(630, B, Hq, Nq, d)
    kp, vp = _rand(631, npages, Hkv, P, d), _rand(632, npages, Hkv, P, d)
    table = np.array([[5, 0, 3], [6, 2, 1]])
    lens = [11, 6]
    O, L = paged(q, kp, vp, table, np.array(lens), P, True, 0.8)
    ok = True
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            for t in range(Nq):
                keys = [j for j in range(lens[b]) if j <= lens[b] - Nq + t]
                row = lambda x, j: [float(c) for c in x[table[b][j // P], h // g, j % P]]
                s = {j: 0.8 * sum(a * c for a, c in zip(q[b, h, t], row(kp, j))) for j in keys}
                mx = max(s.values())
                den = sum(math.exp(s[j] - mx) for j in keys)
                ref = [sum(math.exp(s[j] - mx) / den * row(vp, j)[c] for j in keys) for c in range(d)]
                ok &= np.allclose(O[b, h, t], ref, atol=1e-12, rtol=0) and abs(L[b, h, t] - (mx + math.log(den))) < 1e-12
    return bool(ok)


def check_paged_invariants(paged):
    """Renumbering the physical pages (and the table with them) changes nothing;
    pages the table does not reach, and table entries past a sequence's last
    page, never matter."""
    B, Hq, Hkv, Nq, P, npages, mp, d = 3, 4, 2, 3, 32, 12, 3, 8
    q = _rand(640, B, Hq, Nq, d)
    kp, vp = _rand(641, npages, Hkv, P, d), _rand(642, npages, Hkv, P, d)
    table = np.array([[3, 7, 1], [0, 11, 9], [4, 2, 8]])
    lens = np.array([96, 40, 33])
    O, L = paged(q, kp, vp, table, lens, P, True, 0.3)
    perm = np.random.Generator(np.random.PCG64(643)).permutation(npages)   # physical page i -> perm[i]
    kq, vq = np.empty_like(kp), np.empty_like(vp)
    kq[perm], vq[perm] = kp, vp
    O2, L2 = paged(q, kq, vq, perm[table], lens, P, True, 0.3)
    ok = np.array_equal(O, O2) and np.array_equal(L, L2)
    used = {int(table[b, p]) for b in range(B) for p in range(-(-int(lens[b]) // P))}
    k3, v3, t3 = kp.copy(), vp.copy(), table.copy()
    for i in range(npages):
        if i not in used:
            k3[i], v3[i] = np.inf, np.nan
    t3[1, 2] = 5   # past sequence 1's last page (40 keys = 2 pages)
    O3, L3 = paged(q, k3, v3, t3, lens, P, True, 0.3)
    ok &= np.array_equal(O, O3) and np.array_equal(L, L3)
    return bool(ok)


def paged_oracle(q, kp, vp, table, lens, page_size, causal, scale):
    return oracle.ref_decode_paged(q, kp, vp, table, lens, page_size, causal=causal, scale=scale)


def test_paged_contiguous_case():
    assert check_paged_contiguous_case(paged_oracle)


def test_paged_brute_force():
    assert check_paged_brute_force(paged_oracle)


def test_paged_invariants():
    assert check_paged_invariants(paged_oracle)


# ---------------------------------------------------------------------------
# FP8 forward (thienlv.com glossary, section "Flash Attention 2 và 3": FP8
# support; the format is the OCP FP8 E4M3 definition)
# ---------------------------------------------------------------------------

def check_e4m3_decoder(decode):
    """Values fixed by the format: 1.0 = 0x38, the largest finite 448 = 0x7E, the
    smallest normal 2^-6 = 0x08, the smallest subnormal 2^-9 = 0x01, NaN at 0x7F
    and 0xFF, sign in bit 7; and agreement on every code with the input
    generator's independently written table (round trip of its encoder)."""
    v = decode(np.arange(256))
    ok = v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9
    ok &= bool(np.isnan(v[0x7F]) and np.isnan(v[0xFF])) and v[0x00] == 0.0 and np.signbit(v[0x80])
    ok &= v[0xB8] == -1.0 and v[0x3F] == 1.875 and v[0x40] == 2.0 and v[0x07] == 7 * 2.0 ** -9
    fin = np.r_[0:0x7F, 0x80:0xFF]
    ok &= np.array_equal(W.f32_to_e4m3_bits(v[fin]), fin.astype(np.uint8))
    ok &= np.array_equal(v[fin], W.e4m3_bits_to_f32(fin.astype(np.uint8)).astype(np.float64))
    return bool(ok)


def check_fp8_forward(fwd8, decode):
    """Brute force on tiny inputs through the generator's decoder, and the
    descale invariants: O is linear in the V descale, LSE does not see it;
    moving a factor between the Q and K descales changes nothing."""
    ok = True
    g = np.random.Generator(np.random.PCG64(700))
    for (B, Hq, Hkv, Nq, Nk, d, causal) in [(1, 2, 1, 4, 6, 4, True), (2, 2, 2, 3, 5, 8, False)]:
        q8 = g.integers(0, 256, (B, Hq, Nq, d)).astype(np.uint8) & 0x77   # finite codes of magnitude < 2
        k8 = g.integers(0, 256, (B, Hkv, Nk, d)).astype(np.uint8) & 0x77
        v8 = g.integers(0, 256, (B, Hkv, Nk, d)).astype(np.uint8) & 0xF7
        O, L = fwd8(q8, k8, v8, 0.5, 0.25, 2.0, causal, 0.3)
        qv, kv, vv = (W.e4m3_bits_to_f32(x).astype(np.float64) for x in (q8, k8, v8))
        Ob, Lb = brute_attention(qv * 0.5, kv * 0.25, vv * 2.0, causal, 0.3)
        ok &= np.allclose(O, Ob, atol=1e-12, rtol=0) and np.allclose(L, Lb, atol=1e-12, rtol=0)
        O2, L2 = fwd8(q8, k8, v8, 0.5, 0.25, 8.0, causal, 0.3)
        ok &= np.allclose(O2, 4.0 * O, atol=1e-12) and np.array_equal(L2, L)
        O3, L3 = fwd8(q8, k8, v8, 2.0, 0.0625, 2.0, causal, 0.3)
        ok &= np.allclose(O3, O, atol=1e-12) and np.allclose(L3, L, atol=1e-12)
    return bool(ok)


def fp8_oracle(q8, k8, v8, dq, dk, dv, causal, scale):
    return oracle.ref_fwd_fp8(q8, k8, v8, dq, dk, dv, causal=causal, scale=scale)


def test_e4m3_decoder():
    assert check_e4m3_decoder(oracle.e4m3_value)


def test_fp8_forward():
    assert check_fp8_forward(fp8_oracle, oracle.e4m3_value)
