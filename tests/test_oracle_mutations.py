"""Planted mistakes in the oracle must fail at least one pin.

Each mutant patches one internal step of ``oracle.attention`` (on the CPU) the
way a plausible bug would: a dropped scale, a transposed operand, a wrong
causal offset, softmax over the wrong axis, a dropped term in the logsumexp, the
wrong GQA head map, and the per-block normalisation of the tiled listing in the
holysheep.ai article (section 2.2 "Tiling"), which divides by a block-local sum
at every step and again at the end.  The pins of ``test_oracle_pins`` are then
re-run against the mutated oracle; at least one of them must fail.
"""
import numpy as np
import pytest

import oracle
import oracle.attention as A
import test_oracle_pins as pins

_orig = {n: getattr(A, n) for n in ("scores", "masked_softmax", "valid_mask", "kv_head", "tiled_fwd", "ref_bwd")}


def _fwd_checks():
    fwd = pins.fwd_oracle
    return [lambda: pins.check_brute_force(fwd), lambda: pins.check_closed_forms(fwd),
            lambda: pins.check_invariants(fwd), lambda: pins.check_chunked_equals_one_shot(fwd),
            lambda: pins.check_torch_sdpa(fwd), pins.check_rows_sum_to_one]


def _bwd_checks():
    bwd = pins.bwd_oracle
    return [lambda: pins.check_finite_differences(bwd), lambda: pins.check_gradient_identities(bwd),
            lambda: pins.check_torch_autograd(bwd)]


def _some_check_fails(checks):
    for c in checks:
        try:
            if not c():
                return True
        except Exception:
            return True
    return False


def _softmax_no_lse_max(S, mask):
    P, m, lse = _orig["masked_softmax"](S, mask)
    return P, m, np.where(np.isfinite(lse), lse - np.where(np.isfinite(m), m, 0), lse)


def _softmax_wrong_axis(S, mask):
    P, m, lse = _orig["masked_softmax"](S.T.copy(), mask.T.copy()) if S.shape[0] == S.shape[1] else \
        _orig["masked_softmax"](S, mask)
    if S.shape[0] == S.shape[1]:
        return P.T.copy(), m, lse
    # non-square: normalise columns instead of rows
    E = np.where(mask, np.exp(S - S.max()), 0.0)
    return E / np.maximum(E.sum(axis=0, keepdims=True), 1e-300), m, lse


def _tiled_holysheep_bug(q2, k2, v2, block_q, block_k, causal=False, scale=None, dtype=np.float64):
    """The article's per-block normalisation: O is divided by the current block's sum at each step."""
    q2, k2, v2 = (np.asarray(x, dtype=dtype) for x in (q2, k2, v2))
    Nq, d = q2.shape
    Nk = k2.shape[0]
    scale = scale if scale is not None else 1 / np.sqrt(d)
    O = np.zeros((Nq, d)); L = np.zeros(Nq)
    with np.errstate(all="ignore"):
        return _holysheep_loop(q2, k2, v2, block_q, block_k, causal, scale, O, L, Nq, Nk, d)


def _holysheep_loop(q2, k2, v2, block_q, block_k, causal, scale, O, L, Nq, Nk, d):
    for i0 in range(0, Nq, block_q):
        i1 = min(Nq, i0 + block_q)
        Ob = np.zeros((i1 - i0, d)); mb = np.full(i1 - i0, -np.inf); lb = np.zeros(i1 - i0)
        for j0 in range(0, Nk, block_k):
            j1 = min(Nk, j0 + block_k)
            S = (q2[i0:i1] @ k2[j0:j1].T) * scale
            if causal:
                S = np.where(np.arange(j0, j1)[None] <= np.arange(i0, i1)[:, None] + Nk - Nq, S, -np.inf)
            mn = np.maximum(mb, S.max(axis=1))
            Pb = np.exp(S - mn[:, None])
            ln = Pb.sum(axis=1)
            Ob = (np.exp(mb - mn)[:, None] * Ob + Pb @ v2[j0:j1]) / ln[:, None]
            mb, lb = mn, ln
        O[i0:i1] = Ob / lb[:, None]
        L[i0:i1] = mb + np.log(lb)
    return O, L


def _bwd_no_delta(q, k, v, do, causal=False, scale=None, kv_lens=None):
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    scale = scale if scale is not None else 1 / np.sqrt(d)
    dQ, dK, dV = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        mask = A.valid_mask(Nq, Nk, causal)
        for h in range(Hq):
            g = A.kv_head(h, Hq, Hkv)
            P = A.masked_softmax(A.scores(q[b, h], k[b, g], scale), mask)[0]
            dV[b, g] += P.T @ do[b, h]
            dS = P * (do[b, h] @ v[b, g].T)          # D term dropped
            dQ[b, h] = scale * (dS @ k[b, g])
            dK[b, g] += scale * (dS.T @ q[b, h])
    return dQ, dK, dV


def _bwd_transposed_dv(q, k, v, do, causal=False, scale=None, kv_lens=None):
    dQ, dK, dV = _orig["ref_bwd"](q, k, v, do, causal=causal, scale=scale)
    q64, k64, do64 = (np.asarray(x, dtype=np.float64) for x in (q, k, do))
    B, Hq, Nq, d = q64.shape
    Hkv, Nk = k64.shape[1], k64.shape[2]
    scale = scale if scale is not None else 1 / np.sqrt(d)
    dV = np.zeros_like(dV)
    for b in range(B):
        for h in range(Hq):
            g = A.kv_head(h, Hq, Hkv)
            P = A.masked_softmax(A.scores(q64[b, h], k64[b, g], scale), A.valid_mask(Nq, Nk, causal))[0]
            dV[b, g] += (P @ do64[b, h]) if Nq == Nk else (P.T @ do64[b, h])[::-1]
    return dQ, dK, dV


def _bwd_unscaled_dk(q, k, v, do, causal=False, scale=None, kv_lens=None):
    dQ, dK, dV = _orig["ref_bwd"](q, k, v, do, causal=causal, scale=scale)
    s = scale if scale is not None else 1 / np.sqrt(np.shape(q)[-1])
    return dQ, dK / s, dV


FWD_MUTANTS = {
    "scale_dropped": ("scores", lambda q, k, s: _orig["scores"](q, k, 1.0)),
    "k_transposed_role": ("scores", lambda q, k, s: _orig["scores"](k, q, s).T if q.shape == k.shape
                          else _orig["scores"](q, k[::-1], s)),
    "causal_offset_sign": ("valid_mask", lambda Nq, Nk, c, kv=None: _orig["valid_mask"](Nq, Nk, False, kv) & (
        (np.arange(Nk)[None] <= np.arange(Nq)[:, None] - (Nk - Nq)) if c else True)),
    "causal_strict": ("valid_mask", lambda Nq, Nk, c, kv=None: _orig["valid_mask"](Nq, Nk, False, kv) & (
        (np.arange(Nk)[None] < np.arange(Nq)[:, None] + (Nk - Nq)) | (np.arange(Nk)[None] == 0) if c else True)),
    "lse_without_max": ("masked_softmax", _softmax_no_lse_max),
    "softmax_wrong_axis": ("masked_softmax", _softmax_wrong_axis),
    "gqa_modulo_map": ("kv_head", lambda h, Hq, Hkv: h % Hkv),
    "holysheep_block_normaliser": ("tiled_fwd", _tiled_holysheep_bug),
}

BWD_MUTANTS = {
    "delta_term_dropped": ("ref_bwd", _bwd_no_delta),
    "dv_transposed_operand": ("ref_bwd", _bwd_transposed_dv),
    "dk_scale_dropped": ("ref_bwd", _bwd_unscaled_dk),
}


def test_unmutated_oracle_passes_every_check():
    assert not _some_check_fails(_fwd_checks())
    assert not _some_check_fails(_bwd_checks())


@pytest.mark.parametrize("name", sorted(FWD_MUTANTS))
def test_forward_mutant_is_caught(name, monkeypatch):
    attr, fn = FWD_MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    if attr == "tiled_fwd":
        monkeypatch.setattr(oracle, "tiled_fwd", fn)
    assert _some_check_fails(_fwd_checks()), f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name, monkeypatch):
    attr, fn = BWD_MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    assert _some_check_fails(_bwd_checks()), f"mutant {name} passed every pin"


# chunk decode: plausible slips in the causal offset of the new tokens
def _chunk_offset(shift, from_nmax=False):
    def chunk(q, k, v, lens, causal, scale):
        B, Hq, Nq, d = np.shape(q)
        Nmax = np.shape(k)[2]
        O = np.zeros((B, Hq, Nq, d)); L = np.full((B, Hq, Nq), -np.inf)
        for b in range(B):
            n = int(lens[b])
            for t in range(Nq):
                lim = (Nmax if from_nmax else n) - (Nq - 1 - t) + shift if causal else n
                lim = max(0, min(n, lim))
                Ot, Lt = oracle.ref_fwd(q[b:b + 1, :, t:t + 1], k[b:b + 1, :, :lim], v[b:b + 1, :, :lim], scale=scale)
                O[b, :, t] = Ot[0, :, 0]; L[b, :, t] = Lt[0, :, 0]
        return O, L
    return chunk


CHUNK_MUTANTS = {
    "chunk_sees_next_token": _chunk_offset(+1),
    "chunk_misses_own_token": _chunk_offset(-1),
    "chunk_aligned_to_cache_capacity": _chunk_offset(0, from_nmax=True),
}


def _chunk_checks(chunk):
    return [lambda: pins.check_chunk_brute_force(chunk), lambda: pins.check_chunk_rows_are_decodes(chunk),
            lambda: pins.check_chunk_special_cases(chunk)]


def test_unmutated_chunk_oracle_passes():
    assert not _some_check_fails(_chunk_checks(pins.chunk_oracle))
    # the mutant scaffold with no slip is the oracle itself
    assert not _some_check_fails(_chunk_checks(_chunk_offset(0)))


@pytest.mark.parametrize("name", sorted(CHUNK_MUTANTS))
def test_chunk_mutant_is_caught(name):
    assert _some_check_fails(_chunk_checks(CHUNK_MUTANTS[name])), f"mutant {name} passed every pin"


# paged cache: plausible slips in the page lookup
def _paged_with_gather(gather):
    def paged(q, kp, vp, table, lens, P, causal, scale):
        q = np.asarray(q, dtype=np.float64)
        B, Hq, Nq, d = q.shape
        O = np.zeros((B, Hq, Nq, d)); L = np.full((B, Hq, Nq), -np.inf)
        for b in range(B):
            n = max(0, min(np.shape(table)[1] * P, int(lens[b])))
            kb, vb = gather(kp, table, b, n, P)[None], gather(vp, table, b, n, P)[None]
            O[b:b + 1], L[b:b + 1] = oracle.ref_decode_chunk(q[b:b + 1], kb, vb, [n], causal=causal, scale=scale)
        return O, L
    return paged


def _gather_row_page_swapped(pages, table, b, n, P):
    pages = np.asarray(pages, dtype=np.float64)
    out = np.zeros((pages.shape[1], n, pages.shape[3]))
    for j in range(n):
        out[:, j] = pages[int(table[b, min(j % P, table.shape[1] - 1)]), :, min(j // P, P - 1)]
    return out


def _gather_table_by_page_then_seq(pages, table, b, n, P):
    pages = np.asarray(pages, dtype=np.float64)
    flat = np.asarray(table).T.reshape(table.shape)   # rows read in the wrong order
    out = np.zeros((pages.shape[1], n, pages.shape[3]))
    for j in range(n):
        out[:, j] = pages[int(flat[b, j // P]), :, j % P]
    return out


def _gather_first_page_only(pages, table, b, n, P):
    pages = np.asarray(pages, dtype=np.float64)
    out = np.zeros((pages.shape[1], n, pages.shape[3]))
    for j in range(n):
        out[:, j] = pages[int(table[b, 0]), :, j % P]
    return out


PAGED_MUTANTS = {
    "page_and_row_swapped": _paged_with_gather(_gather_row_page_swapped),
    "table_read_transposed": _paged_with_gather(_gather_table_by_page_then_seq),
    "first_page_reused": _paged_with_gather(_gather_first_page_only),
}


def _paged_checks(paged):
    return [lambda: pins.check_paged_contiguous_case(paged), lambda: pins.check_paged_brute_force(paged),
            lambda: pins.check_paged_invariants(paged)]


def test_unmutated_paged_oracle_passes():
    assert not _some_check_fails(_paged_checks(pins.paged_oracle))
    assert not _some_check_fails(_paged_checks(_paged_with_gather(oracle.gather_pages)))


@pytest.mark.parametrize("name", sorted(PAGED_MUTANTS))
def test_paged_mutant_is_caught(name):
    assert _some_check_fails(_paged_checks(PAGED_MUTANTS[name])), f"mutant {name} passed every pin"


# FP8: plausible slips in the E4M3 decoding and the descales
def _decode_bias8(bits):
    return oracle.e4m3_value(bits) * 0.5


def _decode_subnormal_as_normal(bits):
    b = np.asarray(bits).astype(np.int64)
    v = oracle.e4m3_value(bits)
    e, m = (b >> 3) & 0xF, b & 7
    return np.where((e == 0) & (m > 0), np.where(b >> 7, -1.0, 1.0) * (1 + m / 8.0) * 2.0 ** -7, v)


def _decode_nan_as_finite(bits):
    b = np.asarray(bits).astype(np.int64)
    return np.where((b & 0x7F) == 0x7F, np.where(b >> 7, -480.0, 480.0), oracle.e4m3_value(bits))


def _fp8_with_decoder(decode):
    def fwd8(q8, k8, v8, dq, dk, dv, causal, scale):
        return oracle.ref_fwd(decode(q8) * dq, decode(k8) * dk, decode(v8) * dv, causal=causal, scale=scale)
    return fwd8


def _fp8_descale_v_dropped(q8, k8, v8, dq, dk, dv, causal, scale):
    return oracle.ref_fwd_fp8(q8, k8, v8, dq, dk, 1.0, causal=causal, scale=scale)


FP8_MUTANTS = {
    "decoder_bias_8": (_decode_bias8, _fp8_with_decoder(_decode_bias8)),
    "decoder_subnormal_as_normal": (_decode_subnormal_as_normal, _fp8_with_decoder(_decode_subnormal_as_normal)),
    "decoder_nan_as_finite": (_decode_nan_as_finite, _fp8_with_decoder(_decode_nan_as_finite)),
    "descale_v_dropped": (oracle.e4m3_value, _fp8_descale_v_dropped),
}


def _fp8_checks(decode, fwd8):
    return [lambda: pins.check_e4m3_decoder(decode), lambda: pins.check_fp8_forward(fwd8, decode)]


def test_unmutated_fp8_oracle_passes():
    assert not _some_check_fails(_fp8_checks(oracle.e4m3_value, pins.fp8_oracle))


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_mutant_is_caught(name):
    assert _some_check_fails(_fp8_checks(*FP8_MUTANTS[name])), f"mutant {name} passed every pin"


# ref_fwd_rows: slips in the per-row key range or the head map
def _rows_mutant(limit, head=None):
    def rows_fn(q, k, v, rows, causal, scale):
        B, Hq, Nq, d = np.shape(q)
        Hkv, Nk = np.shape(k)[1], np.shape(k)[2]
        O = np.zeros((len(rows), d)); L = np.full(len(rows), -np.inf)
        for r, (b, h, i) in enumerate(rows):
            g = head(h, Hq, Hkv) if head else h // (Hq // Hkv)
            hi = max(0, min(Nk, limit(i, Nq, Nk))) if causal else Nk
            if hi == 0:
                continue
            s = scale * (k[b, g, :hi] @ q[b, h, i])
            e = np.exp(s - s.max())
            O[r] = e @ v[b, g, :hi] / e.sum(); L[r] = s.max() + np.log(e.sum())
        return O, L
    return rows_fn


ROWS_MUTANTS = {
    "rows_offset_sign_flipped": _rows_mutant(lambda i, Nq, Nk: i - (Nk - Nq) + 1),
    "rows_diagonal_key_dropped": _rows_mutant(lambda i, Nq, Nk: i + (Nk - Nq)),
    "rows_top_left_aligned": _rows_mutant(lambda i, Nq, Nk: i + 1),
    "rows_head_map_interleaved": _rows_mutant(lambda i, Nq, Nk: i + (Nk - Nq) + 1, head=lambda h, Hq, Hkv: h % Hkv),
}


def test_unmutated_rows_oracle_passes():
    assert pins.check_rows_variant(pins.rows_oracle)
    # the mutant scaffold itself, with the right range and head map, passes too
    assert pins.check_rows_variant(_rows_mutant(lambda i, Nq, Nk: i + (Nk - Nq) + 1))


@pytest.mark.parametrize("name", sorted(ROWS_MUTANTS))
def test_rows_mutant_is_caught(name):
    assert not pins.check_rows_variant(ROWS_MUTANTS[name]), f"mutant {name} passed the pin"


# compare: a wrong norm, a signed maximum, the wrong denominator, a lost
# non-finite check
def _cmp_mutant(kind):
    def cmp(gpu, ref):
        g, r = np.asarray(gpu, dtype=np.float64), np.asarray(ref, dtype=np.float64)
        if g.shape != r.shape:
            raise ValueError("shape")
        fin = np.isfinite(r)
        if kind != "nonfinite_ignored":
            if not np.array_equal(np.isfinite(g), fin) or not np.array_equal(g[~fin], r[~fin]):
                return {"max_abs": np.inf, "rel_l2": np.inf, "nonfinite_mismatch": True}
        diff = g[fin] - r[fin]
        nr = np.linalg.norm(r[fin])
        mx = float(np.abs(diff).max()) if diff.size else 0.0
        if kind == "signed_max":
            mx = float(diff.max()) if diff.size else 0.0
        num = np.linalg.norm(diff)
        if kind == "l1_norm":
            num, nr = np.abs(diff).sum(), np.abs(r[fin]).sum()
        if kind == "squared_ratio":
            num, nr = num ** 2, nr ** 2
        if kind == "relative_to_result":
            nr = np.linalg.norm(g[fin])
        return {"max_abs": mx, "rel_l2": float(num / nr) if nr > 0 else float(num)}
    return cmp


COMPARE_MUTANTS = ["signed_max", "l1_norm", "squared_ratio", "relative_to_result", "nonfinite_ignored"]


def test_unmutated_compare_scaffold_passes():
    assert pins.check_compare(_cmp_mutant("none"))


@pytest.mark.parametrize("name", COMPARE_MUTANTS)
def test_compare_mutant_is_caught(name):
    with np.errstate(all="ignore"):
        assert not pins.check_compare(_cmp_mutant(name)), f"mutant {name} passed the pin"
