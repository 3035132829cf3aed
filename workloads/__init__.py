"""Seeded synthetic inputs for the attention workloads.

This module is shared by the CPU oracle (``oracle/``), the tests and the
benchmark.  It holds no attention arithmetic: it only draws random numbers,
rounds them to bfloat16 on the host, and picks the structural choices of each
workload (outlier key rows, sampled query rows, per-sequence cache lengths).

Every stream is ``numpy.random.Generator(PCG64(SeedSequence([42, cfg, t])))``
with base seed 42 (the seed the pages' own examples use), ``cfg`` the workload
id and ``t`` the tensor stream:

    0 Q, 1 K, 2 V, 3 dO, 4 outlier key rows, 5 sampled query rows, 6 lengths,
    7 further query rows for timing the CPU oracle.

Values are ``standard_normal(float32)`` rounded to bfloat16 with
round-to-nearest-even, so the GPU path and the oracle read the same bits.

Workloads (sizes as stated by the five benchmark configurations):

    1  single head, non-causal forward  B1 H1 N256 d64, fp32
    2  causal forward                   B4 H16 N2048 d64, bf16
    3  LLaMA-shaped causal forward      B2 H32 N8192 d128, bf16, 1% K rows x8
    4  GQA decode against a KV cache    B16 Hq32 Hkv8 Nmax32768 d128, bf16,
                                        lengths ~ U{4096..32768}
    5  causal forward + backward        B2 H16 N4096 d128, bf16

``to_fp8`` turns any of them into per-tensor scaled FP8 E4M3 inputs.

``hash_values`` builds inputs too large to draw and copy from the host: an
integer hash of each element's (row, column) index, evaluated on the device
and re-evaluated on the host for any row the oracle needs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 42

STREAM_Q, STREAM_K, STREAM_V, STREAM_DO = 0, 1, 2, 3
STREAM_OUTLIER, STREAM_ROWS, STREAM_LENS, STREAM_MORE_ROWS = 4, 5, 6, 7


def rng(cfg: int, stream: int) -> np.random.Generator:
    """The generator of one tensor stream of one workload."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, int(cfg), int(stream)])))


# ---------------------------------------------------------------------------
# bfloat16 bit handling (host side, round-to-nearest-even)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    NaN stays NaN (quiet), +-inf stays +-inf.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r = r.copy()
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(gen: np.random.Generator, shape) -> np.ndarray:
    return gen.standard_normal(size=shape, dtype=np.float32)


def normal_bf16_bits(gen: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """N(0,1) draws rounded to bfloat16, produced in chunks to bound host memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = f32_to_bf16_bits(gen.standard_normal(size=e - s, dtype=np.float32))
    return out.reshape(shape)


# ---------------------------------------------------------------------------
# FP8 E4M3 (OCP "E4M3FN": 1 sign, 4 exponent bits with bias 7, 3 mantissa
# bits; no infinities; S.1111.111 is NaN; largest finite 448; subnormals
# m * 2^-9).  Host-side encoding of float32 inputs with a per-tensor scale.
# ---------------------------------------------------------------------------

def _e4m3_positive_values() -> np.ndarray:
    """Values of the finite non-negative codes 0x00 .. 0x7E, increasing."""
    c = np.arange(0x7F)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3 value (ties to the even code), saturating at
    +-448; NaN -> 0x7F.  Returns uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    pos = _e4m3_positive_values()
    ax = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(pos, ax), 1, len(pos) - 1)
    lo = hi - 1
    dlo, dhi = ax - pos[lo], pos[hi] - ax
    code = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(ax == 0, 0, code).astype(np.uint8)
    code = code | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def e4m3_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact value of each E4M3 code (NaN for the two NaN codes)."""
    b = np.asarray(bits, dtype=np.uint8)
    pos = np.append(_e4m3_positive_values(), np.nan)
    v = pos[b & 0x7F]
    return np.where(b & 0x80, -v, v).astype(np.float32)


def fp8_quantize(x: np.ndarray):
    """Per-tensor scaled E4M3: codes of x / s and the descale s, a power of two
    with max|x| / s <= 448 (s = 1 for an all-zero tensor)."""
    amax = float(np.max(np.abs(x))) if np.size(x) else 0.0
    s = 2.0 ** math.ceil(math.log2(amax / 448.0)) if amax > 0 else 1.0
    return f32_to_e4m3_bits(np.asarray(x, dtype=np.float64) / s), s


# ---------------------------------------------------------------------------
# Workload descriptions
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    """One synthetic workload.

    Tensors are stored as they enter the library: ``*_bits`` uint16 arrays for
    bf16 workloads, float32 arrays for fp32 ones.  ``values(name)`` returns the
    exact float32 values of either kind.
    """
    cfg: int
    name: str
    dtype: str                      # "bf16" | "f32"
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    decode: bool = False
    tensors: dict = field(default_factory=dict)
    seqlens: np.ndarray | None = None      # decode: int32 [B]
    sample_rows: np.ndarray | None = None  # int64 [R, 3] (b, h, i)
    outlier_rows: np.ndarray | None = None  # int64 [B, Hkv, n_out]

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def values(self, name: str) -> np.ndarray:
        t = self.tensors[name]
        if t.dtype == np.uint16:
            return bf16_bits_to_f32(t)
        return t


CONFIG_NAMES = {
    1: "single_head_noncausal_fwd_B1_H1_N256_d64_f32",
    2: "causal_fwd_B4_H16_N2048_d64_bf16",
    3: "llama_causal_fwd_B2_H32_N8192_d128_bf16_kout",
    4: "gqa_decode_B16_Hq32_Hkv8_N32768_d128_bf16",
    5: "causal_fwd_bwd_B2_H16_N4096_d128_bf16",
}


def _qkv(cfg, dtype, B, Hq, Hkv, Nq, Nk, d, with_do=False):
    t = {}
    shapes = {"q": (B, Hq, Nq, d), "k": (B, Hkv, Nk, d), "v": (B, Hkv, Nk, d)}
    if with_do:
        shapes["do"] = (B, Hq, Nq, d)
    streams = {"q": STREAM_Q, "k": STREAM_K, "v": STREAM_V, "do": STREAM_DO}
    for name, shp in shapes.items():
        g = rng(cfg, streams[name])
        if dtype == "bf16":
            t[name] = normal_bf16_bits(g, shp)
        else:
            t[name] = normal_f32(g, shp)
    return t


def outlier_key_rows(cfg: int, B: int, H: int, N: int, frac: float = 0.01) -> np.ndarray:
    """Per (b, h): round(frac*N) distinct key indices, uniform without replacement."""
    g = rng(cfg, STREAM_OUTLIER)
    n_out = int(round(frac * N))
    rows = np.empty((B, H, n_out), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            rows[b, h] = np.sort(g.choice(N, size=n_out, replace=False))
    return rows


def sampled_query_rows(cfg: int, B: int, H: int, N: int, count: int = 512) -> np.ndarray:
    """``count`` distinct (b, h, i) triples drawn uniformly over all query rows."""
    g = rng(cfg, STREAM_ROWS)
    flat = np.sort(g.choice(B * H * N, size=count, replace=False))
    b = flat // (H * N)
    h = (flat // N) % H
    i = flat % N
    return np.stack([b, h, i], axis=1).astype(np.int64)


def more_query_rows(cfg: int, B: int, H: int, N: int, count: int) -> np.ndarray:
    """Further (b, h, i) triples, uniform over all query rows (with repeats
    possible), from their own stream: the rows the CPU oracle is timed on
    beyond the parity sample."""
    g = rng(cfg, STREAM_MORE_ROWS)
    flat = g.integers(0, B * H * N, size=count, dtype=np.int64)
    return np.stack([flat // (H * N), (flat // N) % H, flat % N], axis=1).astype(np.int64)


def cache_lengths(cfg: int, B: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence valid cache lengths, integers uniform on [lo, hi] inclusive."""
    g = rng(cfg, STREAM_LENS)
    return g.integers(lo, hi + 1, size=B, dtype=np.int64).astype(np.int32)


def make_config(cfg: int, **override) -> Workload:
    """Build workload ``cfg`` (1..5).  ``override`` may shrink B/H/N for tests.

    Overrides keep the recipe (distribution, seeding, structure); only sizes change.
    """
    if cfg == 1:
        p = dict(B=1, Hq=1, Hkv=1, Nq=256, Nk=256, d=64, causal=False, dtype="f32")
    elif cfg == 2:
        p = dict(B=4, Hq=16, Hkv=16, Nq=2048, Nk=2048, d=64, causal=True, dtype="bf16")
    elif cfg == 3:
        p = dict(B=2, Hq=32, Hkv=32, Nq=8192, Nk=8192, d=128, causal=True, dtype="bf16")
    elif cfg == 4:
        p = dict(B=16, Hq=32, Hkv=8, Nq=1, Nk=32768, d=128, causal=False, dtype="bf16",
                 len_lo=4096, len_hi=32768)
    elif cfg == 5:
        p = dict(B=2, Hq=16, Hkv=16, Nq=4096, Nk=4096, d=128, causal=True, dtype="bf16")
    else:
        raise ValueError(f"unknown workload {cfg}")
    p.update(override)
    if cfg == 4:
        # the cache capacity and the length range shrink together
        p.setdefault("len_hi", p["Nk"])
        p["len_hi"] = min(p["len_hi"], p["Nk"])
        p["len_lo"] = min(p["len_lo"], p["len_hi"])
    w = Workload(cfg=cfg, name=CONFIG_NAMES[cfg], dtype=p["dtype"], B=p["B"], Hq=p["Hq"],
                 Hkv=p["Hkv"], Nq=p["Nq"], Nk=p["Nk"], d=p["d"], causal=p["causal"],
                 decode=(cfg == 4))
    w.tensors = _qkv(cfg, w.dtype, w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, with_do=(cfg == 5))
    if cfg == 3:
        rows = outlier_key_rows(cfg, w.B, w.Hkv, w.Nk)
        w.outlier_rows = rows
        k = w.tensors["k"]
        kv = bf16_bits_to_f32(k)
        for b in range(w.B):
            for h in range(w.Hkv):
                kv[b, h, rows[b, h]] *= np.float32(8.0)   # power of two: exact in bf16
        w.tensors["k"] = f32_to_bf16_bits(kv)
        w.sample_rows = sampled_query_rows(cfg, w.B, w.Hq, w.Nq, count=min(512, w.B * w.Hq * w.Nq))
    if cfg == 4:
        w.seqlens = cache_lengths(cfg, w.B, p["len_lo"], p["len_hi"])
    return w


def random_case(seed: int, B, Hq, Hkv, Nq, Nk, d, dtype="bf16", with_do=False, cfg_tag=100):
    """Small seeded case for edge-shape tests (same recipe: N(0,1), bf16 RNE)."""
    w = Workload(cfg=cfg_tag, name=f"case_{seed}", dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk,
                 d=d, causal=False)
    t = {}
    shapes = {"q": (B, Hq, Nq, d), "k": (B, Hkv, Nk, d), "v": (B, Hkv, Nk, d)}
    if with_do:
        shapes["do"] = (B, Hq, Nq, d)
    for si, (name, shp) in enumerate(shapes.items()):
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, cfg_tag, seed, si])))
        t[name] = normal_bf16_bits(g, shp) if dtype == "bf16" else normal_f32(g, shp)
    w.tensors = t
    return w


def random_lengths(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, 200, seed])))
    return g.integers(lo, hi + 1, size=B, dtype=np.int64).astype(np.int32)


def to_fp8(w: Workload) -> dict:
    """E4M3 versions of a workload's q, k, v: per-tensor power-of-two scales
    chosen from each tensor's largest magnitude; returns {name: (codes,
    descale)}.  The values the method then sees are codes * descale."""
    return {n: fp8_quantize(w.values(n)) for n in ("q", "k", "v")}


_M32 = 0xFFFFFFFF
_HASH_VALUE = (np.arange(256) - 128) / 64.0


def hash_values(row, col, salt: int):
    """Values in [-2, 2) on the 1/64 grid (exact in bfloat16) from a 32-bit
    hash of (row, column, salt).  The key is a linear mix of the three; the
    murmur3 32-bit finaliser (xor-shift 16, multiply 0x85EBCA6B, xor-shift 13,
    multiply 0xC2B2AE35, xor-shift 16) then spreads it, so rows and columns
    come out as good as independent (a linear key alone leaves the rows nearly
    parallel).  ``row`` and ``col`` are int64 numpy arrays or torch tensors on
    any device (broadcast together); torch works in int64 masked to 32 bits,
    numpy in uint32, and both give the same values.
    Returns float64 for numpy, float32 for torch."""
    if isinstance(row, np.ndarray):
        # uint32 arithmetic wraps modulo 2^32 by itself; the key's row and
        # column parts are formed on the small operands before broadcasting
        u = np.uint32
        with np.errstate(over="ignore"):
            hr = (np.asarray(row) & _M32).astype(u) * u(0x9E3779B1) + u((salt * 0x68E31DA4) & _M32)
            h = hr + (np.asarray(col) & _M32).astype(u) * u(0x7FEB352D)
            h ^= h >> u(16)
            h *= u(0x85EBCA6B)
            h ^= h >> u(13)
            h *= u(0xC2B2AE35)
            h ^= h >> u(16)
        return _HASH_VALUE[(h >> u(8)) & u(0xFF)]
    import torch
    h = (row * 0x9E3779B1 + col * 0x7FEB352D + salt * 0x68E31DA4) & _M32
    h = h ^ (h >> 16)
    h = (h * 0x85EBCA6B) & _M32
    h = h ^ (h >> 13)
    h = (h * 0xC2B2AE35) & _M32
    h = h ^ (h >> 16)
    return (((h >> 8) & 0xFF) - 128).to(torch.float32) / 64.0
