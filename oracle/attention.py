"""CPU oracle for exact attention (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The GPU library never calls it, and it shares no code with the
GPU library: it is plain numpy in float64 that materialises the full score
matrix S and probability matrix P, which is exactly what the GPU kernels avoid.

Sources (web pages; cited by title and section):

* [KV]   handsonai.io, "DL101 chapter 9", section 1.1 "Key/Value Caching":
         attention of a query against the keys/values up to its position,
         softmax(Q K^T / sqrt(d_k)) V, and the cache that grows one token per step.
* [GQA]  same page, sections 3.1 "Multi-Query Attention" and 3.2
         "Grouped-Query Attention": K/V carry fewer heads than Q; contiguous
         groups of query heads share one K/V head; the output has the query's shape.
* [TILE] same page, section 3.3 "FlashAttention": the tiled forward with the
         running max m and denominator l, the correction factor exp(m_old - m_new)
         applied to both l and the partial output, and one division by l at the end.
* [OS]   holysheep.ai Flash Attention article, section 2.1 "Online Softmax":
         safe softmax (subtract the max) and the running max / running
         denominator recurrence whose final pair (m_n, d_n) normalises every term.
* [HBM]  same article, section 1.2 "HBM vs SRAM": standard attention writes S and
         P (N x N) to memory; the method reads Q, K, V and writes O.
* [RC]   thienlv.com glossary "Flash Attention Là Gì?", section "Ba Kỹ Thuật
         Chính", item 2 (recomputation): the backward pass rebuilds P from Q, K, V
         instead of storing it.  The oracle's backward instead keeps its
         materialised P; it is the plain gradient of the forward definition.
* [SPEC] handsonai.io, "DL101 chapter 9", section 1.2 "Speculative Decoding":
         the large model checks a run of drafted tokens in one pass, each of
         them under the rule of [KV] (attending to the keys up to its own
         position).
* [PAGE] unite.ai "What is FlashAttention", section "Nguồn chính để nghiên cứu
         FlashAttention": names vLLM's PagedAttention (a KV cache kept in
         fixed-size pages reached through a per-sequence block table) as where
         the method meets serving; the pages define nothing further.
* [FP8]  same glossary, section "Flash Attention 2 và 3": FlashAttention-3 adds
         FP8 support.  The pages give no format or scaling; the reading here is
         OCP FP8 E4M3 inputs with one descale factor per tensor (the value of a
         code is its E4M3 value times the descale), and the result is exact
         attention of those values.
* [EX]   same glossary, section "Flash Attention Vs các kỹ Thuật Khác", and
         aiunderstanding.org "FlashAttention", section "Wawasan Teknis": the
         result is the same as standard attention, not an approximation.

Readings taken where the pages are silent (each listed with its reason in the
design notes):

* scale is applied once, to raw inputs; the configurations use 1/sqrt(d).
* logsumexp of a row = natural log of sum_j exp(scale * q.k_j) over its valid
  keys, i.e. m + ln(l) in the recurrence's terms.
* causal masking is bottom-right aligned: key j is visible to query i iff
  j <= i + Nk - Nq (equal to the usual lower-triangular mask when Nq == Nk).
* a row with no valid key has O = 0 and LSE = -inf.
* GQA head map: kv head = h // (Hq // Hkv); dK and dV of a kv head are summed
  over its query heads.
* decode: the single query token sees every key j < len_b (no causal term).
* paged cache: pool [num_pages, Hkv, page_size, d]; block_table[b, p] names the
  physical page holding keys p*page_size .. (p+1)*page_size - 1 of sequence b;
  the result is that of the contiguous cache those pages spell out.
* chunk decode: the Nq new tokens are the last Nq of the len_b cached keys, so
  causal token t sees keys j < len_b - (Nq - 1 - t); a token whose range is
  empty (len_b < Nq - t) is a row with no valid key.

Every function here is pinned by tests (closed forms, invariants, brute force,
the printed tiled-vs-standard result of [TILE], and a library special case).
Parity pinned: all functions.  None is marked "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def default_scale(d: int) -> float:
    """1/sqrt(d_k) as in [KV]."""
    return 1.0 / math.sqrt(d)


def valid_mask(Nq: int, Nk: int, causal: bool, kv_len: int | None = None) -> np.ndarray:
    """Boolean [Nq, Nk]: which keys each query row may attend to.

    Key j is valid iff j < kv_len (cache length, [KV]) and, when causal,
    j <= i + Nk - Nq (bottom-right alignment; the newest query sees every key).
    """
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    m = np.ones((Nq, Nk), dtype=bool)
    if kv_len is not None:
        m &= j < int(kv_len)
    if causal:
        m &= j <= i + (Nk - Nq)
    return m


def scores(q_bh: np.ndarray, k_bh: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T for one head, materialised (N x N), [KV] / [HBM]."""
    return scale * (_f64(q_bh) @ _f64(k_bh).T)


def masked_softmax(S: np.ndarray, mask: np.ndarray):
    """Row-wise safe softmax over the valid entries ([OS]: subtract the row max).

    Returns (P, m, lse): P is zero outside the mask; rows with no valid entry get
    P = 0, m = -inf, lse = -inf.
    """
    Sm = np.where(mask, S, NEG_INF)
    any_valid = mask.any(axis=1)
    m = np.where(any_valid, Sm.max(axis=1, initial=NEG_INF), NEG_INF)
    m_safe = np.where(any_valid, m, 0.0)
    E = np.where(mask, np.exp(Sm - m_safe[:, None]), 0.0)
    l = E.sum(axis=1)
    l_safe = np.where(any_valid, l, 1.0)
    P = E / l_safe[:, None]
    lse = np.where(any_valid, m_safe + np.log(l_safe), NEG_INF)
    return P, m, lse


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """[GQA]: contiguous groups of Hq/Hkv query heads share one K/V head."""
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def ref_fwd(q, k, v, causal: bool = False, scale: float | None = None, kv_lens=None):
    """Exact attention forward, materialising S and P per head.

    q [B,Hq,Nq,d]; k, v [B,Hkv,Nk,d]; kv_lens optional [B] valid key counts.
    Returns O [B,Hq,Nq,d] and LSE [B,Hq,Nq] in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if scale is None:
        scale = default_scale(d)
    O = np.zeros((B, Hq, Nq, d))
    LSE = np.full((B, Hq, Nq), NEG_INF)
    for b in range(B):
        # keys at or beyond the cache length are outside every row's valid set;
        # they are left out of the products altogether (their contents may be
        # anything, even NaN, without reaching O)
        n = Nk if kv_lens is None else max(0, min(Nk, int(kv_lens[b])))
        mask = valid_mask(Nq, Nk, causal)[:, :n]
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            S = scores(q[b, h], k[b, g, :n], scale)
            P, _, lse = masked_softmax(S, mask)
            O[b, h] = P @ v[b, g, :n]
            LSE[b, h] = lse
    return O, LSE


def ref_probs(q, k, causal: bool = False, scale: float | None = None, kv_lens=None):
    """The materialised P [B,Hq,Nq,Nk] (small shapes only; used by invariant tests)."""
    q, k = _f64(q), _f64(k)
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if scale is None:
        scale = default_scale(d)
    P = np.zeros((B, Hq, Nq, Nk))
    for b in range(B):
        mask = valid_mask(Nq, Nk, causal, None if kv_lens is None else int(kv_lens[b]))
        for h in range(Hq):
            P[b, h] = masked_softmax(scores(q[b, h], k[b, kv_head(h, Hq, Hkv)], scale), mask)[0]
    return P


def ref_fwd_rows(q, k, v, rows, causal: bool = False, scale: float | None = None):
    """O and LSE for selected query rows only, each against its own valid keys.

    rows: int array [R, 3] of (b, h, i).  Same definition as ref_fwd, one row at
    a time, so a large problem can be checked on a sample of rows.
    """
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if scale is None:
        scale = default_scale(d)
    R = len(rows)
    O = np.zeros((R, d))
    LSE = np.full(R, NEG_INF)
    for r, (b, h, i) in enumerate(np.asarray(rows, dtype=np.int64)):
        g = kv_head(int(h), Hq, Hkv)
        hi = (int(i) + (Nk - Nq) + 1) if causal else Nk
        hi = max(0, min(Nk, hi))
        if hi == 0:
            continue
        kk = _f64(k[b, g, :hi])
        vv = _f64(v[b, g, :hi])
        s = scale * (kk @ _f64(q[b, h, i]))
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        O[r] = (e / l) @ vv
        LSE[r] = m + np.log(l)
    return O, LSE


def ref_decode(q, k_cache, v_cache, seqlens, scale: float | None = None):
    """One new query token per (b, h) against the first seqlens[b] cached keys ([KV]).

    q [B,Hq,1,d]; caches [B,Hkv,Nmax,d]; returns O [B,Hq,1,d], LSE [B,Hq].
    """
    O, LSE = ref_fwd(q, k_cache, v_cache, causal=False, scale=scale, kv_lens=seqlens)
    return O, LSE[:, :, 0]


def ref_decode_chunk(q, k_cache, v_cache, seqlens, causal: bool = True, scale: float | None = None):
    """Nq new query tokens per (b, h) against the first seqlens[b] cached keys,
    of which the last Nq are the new tokens' own ([SPEC], with [KV]'s rule).

    causal: token t sees keys j < seqlens[b] - (Nq - 1 - t), i.e. the forward
    over the sequence's own keys with bottom-right alignment; otherwise every
    token sees keys j < seqlens[b].  q [B,Hq,Nq,d]; caches [B,Hkv,Nmax,d];
    returns O [B,Hq,Nq,d], LSE [B,Hq,Nq].
    """
    q = _f64(q)
    B, Hq, Nq, d = q.shape
    Nmax = np.shape(k_cache)[2]
    O = np.zeros((B, Hq, Nq, d))
    LSE = np.full((B, Hq, Nq), NEG_INF)
    for b in range(B):
        n = max(0, min(Nmax, int(seqlens[b])))
        O[b:b + 1], LSE[b:b + 1] = ref_fwd(q[b:b + 1], _f64(k_cache[b:b + 1, :, :n]), _f64(v_cache[b:b + 1, :, :n]),
                                           causal=causal, scale=scale)
    return O, LSE


def gather_pages(pages, block_table, b: int, n: int, page_size: int) -> np.ndarray:
    """The first n keys of sequence b as a contiguous [Hkv, n, d] array ([PAGE]):
    key j lives in physical page block_table[b, j // page_size], row j % page_size."""
    pages = _f64(pages)
    Hkv, d = pages.shape[1], pages.shape[3]
    out = np.zeros((Hkv, n, d))
    for j in range(n):
        out[:, j] = pages[int(block_table[b, j // page_size]), :, j % page_size]
    return out


def ref_decode_paged(q, k_pages, v_pages, block_table, seqlens, page_size: int, causal: bool = True,
                     scale: float | None = None):
    """Chunk decode (ref_decode_chunk) against a paged cache ([PAGE]).

    k_pages/v_pages [num_pages, Hkv, page_size, d]; block_table [B, max_pages]
    int; seqlens [B] clamped to [0, max_pages * page_size].  q [B,Hq,Nq,d];
    returns O [B,Hq,Nq,d], LSE [B,Hq,Nq].
    """
    q = _f64(q)
    B, Hq, Nq, d = q.shape
    cap = np.shape(block_table)[1] * page_size
    O = np.zeros((B, Hq, Nq, d))
    LSE = np.full((B, Hq, Nq), NEG_INF)
    for b in range(B):
        n = max(0, min(cap, int(seqlens[b])))
        kb = gather_pages(k_pages, block_table, b, n, page_size)[None]
        vb = gather_pages(v_pages, block_table, b, n, page_size)[None]
        O[b:b + 1], LSE[b:b + 1] = ref_decode_chunk(q[b:b + 1], kb, vb, [n], causal=causal, scale=scale)
    return O, LSE


def e4m3_value(bits) -> np.ndarray:
    """Value of OCP FP8 E4M3 codes ([FP8]): sign bit 7, exponent bits 6..3
    (bias 7), mantissa bits 2..0; exponent 0 is subnormal (m * 2^-9); the code
    with every exponent and mantissa bit set is NaN; there is no infinity."""
    b = np.asarray(bits).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m, -9), np.ldexp(8.0 + m, (e - 10).astype(np.int64)))
    return np.where((e == 0xF) & ((b & 0x7) == 0x7), np.nan, sign * mag)


def ref_fwd_fp8(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float, causal: bool = False,
                scale: float | None = None):
    """Exact attention of FP8 inputs ([FP8]): the values are e4m3_value(code) *
    descale per tensor; scale defaults to 1/sqrt(d).  Returns O, LSE (float64)."""
    q = e4m3_value(q8) * float(descale_q)
    k = e4m3_value(k8) * float(descale_k)
    v = e4m3_value(v8) * float(descale_v)
    return ref_fwd(q, k, v, causal=causal, scale=scale)


def ref_bwd(q, k, v, do, causal: bool = False, scale: float | None = None, kv_lens=None):
    """Gradients of sum(O * dO) with respect to Q, K, V (float64).

    Plain chain rule through the materialised forward:
      dV_j = sum_i P_ij dO_i;  dP_ij = dO_i . V_j;  D_i = sum_j P_ij dP_ij;
      dS_ij = P_ij (dP_ij - D_i);  dQ_i = scale sum_j dS_ij K_j;
      dK_j = scale sum_i dS_ij Q_i.
    GQA: dK, dV of a kv head are the sums over its query heads.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if scale is None:
        scale = default_scale(d)
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for b in range(B):
        mask = valid_mask(Nq, Nk, causal, None if kv_lens is None else int(kv_lens[b]))
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            P = masked_softmax(scores(q[b, h], k[b, g], scale), mask)[0]
            dV[b, g] += P.T @ do[b, h]
            dP = do[b, h] @ v[b, g].T
            D = (P * dP).sum(axis=1)
            dS = P * (dP - D[:, None])
            dQ[b, h] = scale * (dS @ k[b, g])
            dK[b, g] += scale * (dS.T @ q[b, h])
    return dQ, dK, dV


# ---------------------------------------------------------------------------
# The method's own recurrence, written from the pages, used to pin the
# definition above (chunked == one-shot) and to define the split merge.
# ---------------------------------------------------------------------------

def online_softmax_stats(chunks):
    """Running (max, denominator) over a sequence of score chunks ([OS]).

    Returns (m_n, d_n) such that softmax(x)_j = exp(x_j - m_n) / d_n.
    """
    m = NEG_INF
    dsum = 0.0
    for c in chunks:
        c = _f64(c)
        if c.size == 0:
            continue
        m_new = max(m, float(c.max()))
        if m_new == NEG_INF:
            continue
        dsum = dsum * math.exp(m - m_new) + float(np.exp(c - m_new).sum())
        m = m_new
    return m, dsum


def tiled_fwd(q2, k2, v2, block_q: int, block_k: int, causal: bool = False,
              scale: float | None = None, dtype=np.float64):
    """The tiled forward of [TILE] for one head, in the given float dtype.

    q2 [Nq,d], k2/v2 [Nk,d].  For each query block: m = -inf, l = 0, O = 0; for
    each key block: S = scale Q K^T, m_new = max(m, rowmax S), P = exp(S - m_new),
    c = exp(m - m_new), l = c l + rowsum P, O = c O + P V; finally O / l.
    Ragged last blocks are handled by slicing (the page's buffers assume full
    blocks).  Masked entries are -inf; a row that has seen no valid key keeps
    m = -inf and contributes nothing.  Returns O and LSE = m + ln l.
    """
    q2 = np.asarray(q2, dtype=dtype)
    k2 = np.asarray(k2, dtype=dtype)
    v2 = np.asarray(v2, dtype=dtype)
    Nq, d = q2.shape
    Nk = k2.shape[0]
    if scale is None:
        scale = default_scale(d)
    scale = dtype(scale)
    O = np.zeros((Nq, d), dtype=dtype)
    LSE = np.full(Nq, NEG_INF, dtype=dtype)
    for i0 in range(0, Nq, block_q):
        i1 = min(Nq, i0 + block_q)
        Qb = q2[i0:i1]
        Ob = np.zeros((i1 - i0, d), dtype=dtype)
        lb = np.zeros((i1 - i0, 1), dtype=dtype)
        mb = np.full((i1 - i0, 1), NEG_INF, dtype=dtype)
        for j0 in range(0, Nk, block_k):
            j1 = min(Nk, j0 + block_k)
            S = (Qb @ k2[j0:j1].T) * scale
            if causal:
                ii = np.arange(i0, i1)[:, None]
                jj = np.arange(j0, j1)[None, :]
                S = np.where(jj <= ii + (Nk - Nq), S, dtype(NEG_INF))
            m_new = np.maximum(mb, S.max(axis=1, keepdims=True))
            m_sub = np.where(np.isneginf(m_new), dtype(0), m_new)
            P = np.exp(S - m_sub)
            corr = np.where(np.isneginf(m_new), dtype(1), np.exp(mb - m_sub))
            lb = lb * corr + P.sum(axis=1, keepdims=True)
            Ob = Ob * corr + P @ v2[j0:j1]
            mb = m_new
        ok = lb[:, 0] > 0
        O[i0:i1] = np.where(ok[:, None], Ob / np.where(lb > 0, lb, 1), 0)
        LSE[i0:i1] = np.where(ok, mb[:, 0] + np.log(np.where(ok, lb[:, 0], 1)), NEG_INF)
    return O, LSE


def merge_partials(o_parts, lse_parts):
    """Merge attention over disjoint key ranges.

    o_parts [S, ..., d] are each range's normalised outputs and lse_parts [S, ...]
    their logsumexps.  The combined normaliser is sum_s exp(lse_s) and each part
    is re-weighted by exp(lse_s - lse): the same rescaling by exp(m_old - m_new)
    that the running recurrence of [OS] applies when a new block arrives.
    Ranges with lse = -inf (no valid key) get weight 0.
    """
    o_parts = _f64(o_parts)
    lse_parts = _f64(lse_parts)
    m = lse_parts.max(axis=0)
    fin = np.isfinite(m)
    m_safe = np.where(fin, m, 0.0)
    w = np.where(np.isneginf(lse_parts), 0.0, np.exp(lse_parts - m_safe))
    tot = w.sum(axis=0)
    tot_safe = np.where(tot > 0, tot, 1.0)
    O = (w[..., None] * o_parts).sum(axis=0) / tot_safe[..., None]
    lse = np.where(tot > 0, m_safe + np.log(tot_safe), NEG_INF)
    return O, lse


# ---------------------------------------------------------------------------
# Comparison metrics used by every parity test
# ---------------------------------------------------------------------------

def compare(gpu, ref):
    """max-abs and rel-L2 in float64 over the whole array.

    max_abs = max |gpu - ref| and rel_l2 = ||gpu - ref||_2 / ||ref||_2 over the
    finite entries of ref (the absolute ||gpu - ref||_2 when ref is all zero).
    Non-finite entries of ref (LSE = -inf of rows that see no key) must be
    matched exactly by gpu, and gpu must be finite wherever ref is: otherwise
    the result is flagged ``nonfinite_mismatch`` with both metrics infinite.
    A NaN anywhere is a mismatch.  Arrays of different shapes raise ValueError.
    """
    g = _f64(gpu)
    r = _f64(ref)
    if g.shape != r.shape:
        raise ValueError(f"compare: shapes differ {g.shape} vs {r.shape}")
    fin = np.isfinite(r)
    if not np.array_equal(np.isfinite(g), fin):
        return {"max_abs": float("inf"), "rel_l2": float("inf"), "nonfinite_mismatch": True}
    if not fin.all():
        # -inf entries (empty rows) must agree exactly
        if not np.array_equal(g[~fin], r[~fin]):
            return {"max_abs": float("inf"), "rel_l2": float("inf"), "nonfinite_mismatch": True}
    diff = g[fin] - r[fin]
    nr = np.linalg.norm(r[fin])
    return {
        "max_abs": float(np.abs(diff).max()) if diff.size else 0.0,
        "rel_l2": float(np.linalg.norm(diff) / nr) if nr > 0 else float(np.linalg.norm(diff)),
    }
