"""Python binding of libfa (exact IO-aware attention on MI355X / gfx950).

Argument marshalling only: every tensor's shape and dtype are checked against
the others' (the C ABI sees only pointers and sizes, so a mismatch here would
otherwise become an out-of-bounds device access), then device and contiguity;
the device pointers and torch's current HIP stream are passed to the C ABI
(``include/fa.h``), and a non-zero status raises ``RuntimeError``.  Shape
mismatches raise ``ValueError``, dtype mismatches ``TypeError``.
Every step of the computation runs in the HIP kernels of ``libfa.so``; there is
no fallback of any kind.  PyTorch only provides device memory and streams.

Low-level entry points mirror the C names (``fa_fwd``, ``fa_bwd``,
``fa_decode``, ``fa_decode_chunk``, ``fa_decode_paged`` and their
``*_workspace_bytes``) and write into caller-provided tensors; the
``prepare_*`` functions do the checks and marshalling once and return a
callable that only launches (for tight loops).  ``fwd``, ``bwd``, ``decode``,
``decode_chunk`` and ``decode_paged`` allocate their outputs with torch and
call them.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_F32, FA_BF16 = 0, 1
FA_OK = 0

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_io_aware_16_amd.build`")
    # torch ships its own HIP runtime and requests it as "libamdhip64.so";
    # libfa requests "libamdhip64.so.7".  Loading torch first lets libfa's
    # request resolve (by SONAME) to torch's copy, so one runtime serves both
    # and torch's stream handles are valid in libfa.  The other order would
    # map two runtimes into the process.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_abi_version.restype = i
    lib.fa_abi_version.argtypes = []
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_status_str.argtypes = [i]
    lib.fa_fwd.restype = i
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_bwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_decode.restype = i
    lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    lib.fa_decode_chunk_workspace_bytes.restype = sz
    lib.fa_decode_chunk_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_decode_chunk.restype = i
    lib.fa_decode_chunk.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, f, f, i, vp]
    lib.fa_decode_noalloc.restype = i
    lib.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_decode_paged_workspace_bytes.restype = sz
    lib.fa_decode_paged_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_decode_paged.restype = i
    lib.fa_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    _lib = lib
    return lib


def _check(status: int):
    if status != FA_OK:
        raise RuntimeError(load_library().fa_status_str(status).decode())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _dev(*tensors):
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _same_dtype(ref, *named):
    for name, t in named:
        if t.dtype != ref.dtype:
            raise TypeError(f"{name} is {t.dtype}, expected {ref.dtype} (the dtype of q)")


def _f32(t, name):
    if t.dtype != _torch().float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")


def _i32(t, name):
    if t.dtype != _torch().int32:
        raise TypeError(f"{name} must be int32, got {t.dtype}")


def _qkv(q, k, v, kname="k", vname="v"):
    """q [B,Hq,Nq,d], k and v [B,Hkv,Nk,d] of one shape; returns the sizes."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-d [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"{kname} {tuple(k.shape)} does not match q {tuple(q.shape)} in batch or head dimension")
    _shape(v, k.shape, vname)
    return B, Hq, Hkv, Nq, Nk, d


def _workspace(ws):
    if ws.dim() < 1:
        raise ValueError("workspace must be a 1-d (or larger) tensor")


def _stream(stream):
    torch = _torch()
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------------------
# C-ABI mirrors
# ---------------------------------------------------------------------------

def fa_abi_version() -> int:
    return load_library().fa_abi_version()


def fa_bwd_workspace_bytes(B, Hq, Nq, d) -> int:
    return load_library().fa_bwd_workspace_bytes(B, Hq, Nq, d)


def fa_decode_workspace_bytes(B, Hq, Hkv, Nmax, d) -> int:
    return load_library().fa_decode_workspace_bytes(B, Hq, Hkv, Nmax, d)


def fa_decode_chunk_workspace_bytes(B, Hq, Hkv, Nq, Nmax, d) -> int:
    return load_library().fa_decode_chunk_workspace_bytes(B, Hq, Hkv, Nq, Nmax, d)


def fa_decode_paged_workspace_bytes(B, Hq, Hkv, Nq, d) -> int:
    return load_library().fa_decode_paged_workspace_bytes(B, Hq, Hkv, Nq, d)


def prepare_fwd(q, k, v, o, lse, causal=False, scale=None, stream=None):
    """Check and marshal the arguments of fa_fwd once; returns a zero-argument
    callable that launches it (the tensors must stay alive and unchanged in
    shape).  Raises on a non-zero status when called."""
    B, Hq, Hkv, Nq, Nk, d = _qkv(q, k, v)
    dcode = _dtype_code(q)
    _same_dtype(q, ("k", k), ("v", v), ("o", o))
    _shape(o, q.shape, "o")
    _f32(lse, "lse")
    _shape(lse, (B, Hq, Nq), "lse")
    _dev(q, k, v, o, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load_library()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, dcode, scale,
            int(bool(causal)), _stream(stream))
    return lambda: _check(lib.fa_fwd(*args))


def prepare_fwd_fp8(q8, k8, v8, o, lse, descale_q, descale_k, descale_v, causal=False, scale=None, stream=None):
    """fa_fwd_fp8's arguments checked and marshalled once.  q8, k8, v8 hold E4M3
    codes (torch.uint8 or torch.float8_e4m3fn); o is bfloat16."""
    torch = _torch()
    codes = (torch.uint8,) + ((torch.float8_e4m3fn,) if hasattr(torch, "float8_e4m3fn") else ())
    if q8.dtype not in codes or k8.dtype not in codes or v8.dtype not in codes:
        raise TypeError("q8, k8, v8 must hold E4M3 codes (uint8 or float8_e4m3fn)")
    if o.dtype != torch.bfloat16:
        raise TypeError("o must be bfloat16")
    B, Hq, Hkv, Nq, Nk, d = _qkv(q8, k8, v8, "k8", "v8")
    _shape(o, q8.shape, "o")
    _f32(lse, "lse")
    _shape(lse, (B, Hq, Nq), "lse")
    _dev(q8, k8, v8, o, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load_library()
    args = (_ptr(q8), _ptr(k8), _ptr(v8), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, float(descale_q),
            float(descale_k), float(descale_v), scale, int(bool(causal)), _stream(stream))
    return lambda: _check(lib.fa_fwd_fp8(*args))


def fa_fwd_fp8(q8, k8, v8, o, lse, descale_q, descale_k, descale_v, causal=False, scale=None, stream=None):
    """Exact attention of E4M3 inputs (value = code value * descale) into bf16 ``o``."""
    prepare_fwd_fp8(q8, k8, v8, o, lse, descale_q, descale_k, descale_v, causal=causal, scale=scale,
                    stream=stream)()


def fa_fwd(q, k, v, o, lse, causal=False, scale=None, stream=None):
    """O = softmax(scale Q K^T [+causal]) V into ``o``; row logsumexp into ``lse``."""
    prepare_fwd(q, k, v, o, lse, causal=causal, scale=scale, stream=stream)()


def prepare_bwd(q, k, v, o, dO, lse, dq, dk, dv, workspace, causal=False, scale=None, stream=None):
    """fa_bwd's arguments checked and marshalled once (see prepare_fwd)."""
    B, Hq, Hkv, Nq, Nk, d = _qkv(q, k, v)
    dcode = _dtype_code(q)
    _same_dtype(q, ("k", k), ("v", v), ("o", o), ("dO", dO))
    _shape(o, q.shape, "o")
    _shape(dO, q.shape, "dO")
    _f32(lse, "lse")
    _shape(lse, (B, Hq, Nq), "lse")
    gcode = _dtype_code(dq)
    if _dtype_code(dk) != gcode or _dtype_code(dv) != gcode:
        raise TypeError("dq, dk, dv must share one dtype")
    if dcode == FA_F32 and gcode != FA_F32:
        raise TypeError("float32 inputs give float32 gradients only")
    _shape(dq, q.shape, "dq")
    _shape(dk, k.shape, "dk")
    _shape(dv, k.shape, "dv")
    _workspace(workspace)
    _dev(q, k, v, o, dO, lse, dq, dk, dv, workspace)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load_library()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), gcode, B, Hq,
            Hkv, Nq, Nk, d, dcode, scale, int(bool(causal)), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    return lambda: _check(lib.fa_bwd(*args))


def fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, workspace, causal=False, scale=None, stream=None):
    """Gradients of sum(O * dO) into dq, dk, dv (their dtype picks the gradient dtype)."""
    prepare_bwd(q, k, v, o, dO, lse, dq, dk, dv, workspace, causal=causal, scale=scale, stream=stream)()


def prepare_decode(q, k_cache, v_cache, seqlens, o, lse, workspace, scale=None, stream=None):
    """fa_decode's arguments checked and marshalled once (see prepare_fwd)."""
    B, Hq, Hkv, one, Nmax, d = _qkv(q, k_cache, v_cache, "k_cache", "v_cache")
    if one != 1:
        raise ValueError(f"q must hold one token per head [B, Hq, 1, d], got {tuple(q.shape)}")
    dcode = _dtype_code(q)
    _same_dtype(q, ("k_cache", k_cache), ("v_cache", v_cache), ("o", o))
    _shape(o, q.shape, "o")
    _f32(lse, "lse")
    if tuple(lse.shape) not in ((B, Hq), (B, Hq, 1)):
        raise ValueError(f"lse has shape {tuple(lse.shape)}, expected {(B, Hq)}")
    _i32(seqlens, "seqlens")
    _shape(seqlens, (B,), "seqlens")
    _workspace(workspace)
    _dev(q, k_cache, v_cache, seqlens, o, lse, workspace)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load_library()
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), _ptr(lse), B, Hq, Hkv, Nmax, d,
            dcode, scale, _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    return lambda: _check(lib.fa_decode(*args))


def fa_decode(q, k_cache, v_cache, seqlens, o, lse, workspace, scale=None, stream=None):
    """One query token per head against the first seqlens[b] cached keys."""
    prepare_decode(q, k_cache, v_cache, seqlens, o, lse, workspace, scale=scale, stream=stream)()


def prepare_decode_noalloc(q, k_cache, v_cache, seqlens, o, lse, scale=None, stream=None):
    """fa_decode_noalloc's arguments checked and marshalled once (see
    prepare_fwd): fa_decode without a workspace, its partial results in the
    library's fixed per-device scratch (calls that overlap on one device race)."""
    B, Hq, Hkv, one, Nmax, d = _qkv(q, k_cache, v_cache, "k_cache", "v_cache")
    if one != 1:
        raise ValueError(f"q must hold one token per head [B, Hq, 1, d], got {tuple(q.shape)}")
    dcode = _dtype_code(q)
    _same_dtype(q, ("k_cache", k_cache), ("v_cache", v_cache), ("o", o))
    _shape(o, q.shape, "o")
    _f32(lse, "lse")
    if tuple(lse.shape) not in ((B, Hq), (B, Hq, 1)):
        raise ValueError(f"lse has shape {tuple(lse.shape)}, expected {(B, Hq)}")
    _i32(seqlens, "seqlens")
    _shape(seqlens, (B,), "seqlens")
    _dev(q, k_cache, v_cache, seqlens, o, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load_library()
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), _ptr(lse), B, Hq, Hkv, Nmax, d,
            dcode, scale, _stream(stream))
    return lambda: _check(lib.fa_decode_noalloc(*args))


def fa_decode_noalloc(q, k_cache, v_cache, seqlens, o, lse, scale=None, stream=None):
    """fa_decode into caller-provided o and lse without a workspace (the
    library's fixed device scratch holds the partial results)."""
    prepare_decode_noalloc(q, k_cache, v_cache, seqlens, o, lse, scale=scale, stream=stream)()


def prepare_decode_chunk(q, k_cache, v_cache, seqlens, o, lse, workspace, causal=True, scale=None, stream=None):
    """fa_decode_chunk's arguments checked and marshalled once (see prepare_fwd)."""
    B, Hq, Hkv, Nq, Nmax, d = _qkv(q, k_cache, v_cache, "k_cache", "v_cache")
    dcode = _dtype_code(q)
    _same_dtype(q, ("k_cache", k_cache), ("v_cache", v_cache), ("o", o))
    _shape(o, q.shape, "o")
    _f32(lse, "lse")
    _shape(lse, (B, Hq, Nq), "lse")
    _i32(seqlens, "seqlens")
    _shape(seqlens, (B,), "seqlens")
    _workspace(workspace)
    _dev(q, k_cache, v_cache, seqlens, o, lse, workspace)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load_library()
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nmax, d,
            dcode, scale, int(bool(causal)), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream))
    return lambda: _check(lib.fa_decode_chunk(*args))


def fa_decode_chunk(q, k_cache, v_cache, seqlens, o, lse, workspace, causal=True, scale=None, stream=None):
    """Nq new tokens per head against the first seqlens[b] cached keys (the last
    Nq of which are theirs); causal: token t sees keys < seqlens[b] - (Nq-1-t)."""
    prepare_decode_chunk(q, k_cache, v_cache, seqlens, o, lse, workspace, causal=causal, scale=scale,
                         stream=stream)()


def prepare_decode_paged(q, k_pages, v_pages, block_table, seqlens, o, lse, workspace, causal=True, scale=None,
                         stream=None):
    """fa_decode_paged's arguments checked and marshalled once (see prepare_fwd).
    k_pages/v_pages [num_pages, Hkv, page_size, d]; block_table [B, max_pages] int32."""
    if q.dim() != 4 or k_pages.dim() != 4:
        raise ValueError("q [B, Hq, Nq, d] and k_pages [num_pages, Hkv, page_size, d] must be 4-d")
    B, Hq, Nq, d = q.shape
    num_pages, Hkv, page_size, dk = k_pages.shape
    if dk != d:
        raise ValueError(f"k_pages {tuple(k_pages.shape)} does not match q {tuple(q.shape)} in head dimension")
    _shape(v_pages, k_pages.shape, "v_pages")
    dcode = _dtype_code(q)
    _same_dtype(q, ("k_pages", k_pages), ("v_pages", v_pages), ("o", o))
    _shape(o, q.shape, "o")
    _f32(lse, "lse")
    _shape(lse, (B, Hq, Nq), "lse")
    _i32(seqlens, "seqlens")
    _shape(seqlens, (B,), "seqlens")
    _i32(block_table, "block_table")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B={B}, max_pages], got {tuple(block_table.shape)}")
    max_pages = block_table.shape[1]
    _workspace(workspace)
    _dev(q, k_pages, v_pages, block_table, seqlens, o, lse, workspace)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load_library()
    args = (_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seqlens), _ptr(o), _ptr(lse), B, Hq,
            Hkv, Nq, num_pages, page_size, max_pages, d, dcode, scale, int(bool(causal)), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    return lambda: _check(lib.fa_decode_paged(*args))


def fa_decode_paged(q, k_pages, v_pages, block_table, seqlens, o, lse, workspace, causal=True, scale=None,
                    stream=None):
    """fa_decode_chunk against a paged cache: key j of sequence b is row
    j % page_size of page block_table[b, j // page_size]."""
    prepare_decode_paged(q, k_pages, v_pages, block_table, seqlens, o, lse, workspace, causal=causal, scale=scale,
                         stream=stream)()


# ---------------------------------------------------------------------------
# allocating conveniences (outputs allocated by torch, computed by libfa)
# ---------------------------------------------------------------------------

def fwd(q, k, v, causal=False, scale=None, stream=None):
    torch = _torch()
    B, Hq, Nq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, causal=causal, scale=scale, stream=stream)
    return o, lse


def bwd(q, k, v, o, dO, lse, causal=False, scale=None, grad_dtype=None, stream=None):
    torch = _torch()
    B, Hq, Nq, d = q.shape
    gd = torch.float32 if grad_dtype is None else grad_dtype
    dq = torch.empty(q.shape, dtype=gd, device=q.device)
    dk = torch.empty(k.shape, dtype=gd, device=q.device)
    dv = torch.empty(v.shape, dtype=gd, device=q.device)
    ws = torch.empty(max(1, fa_bwd_workspace_bytes(B, Hq, Nq, d)), dtype=torch.uint8, device=q.device)
    fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, ws, causal=causal, scale=scale, stream=stream)
    return dq, dk, dv


def decode_workspace(q, k_cache):
    torch = _torch()
    B, Hq, _, d = q.shape
    _, Hkv, Nmax, _ = k_cache.shape
    return torch.empty(max(1, fa_decode_workspace_bytes(B, Hq, Hkv, Nmax, d)), dtype=torch.uint8,
                       device=q.device)


def decode(q, k_cache, v_cache, seqlens, scale=None, workspace=None, stream=None):
    torch = _torch()
    B, Hq, _, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ws = decode_workspace(q, k_cache) if workspace is None else workspace
    fa_decode(q, k_cache, v_cache, seqlens, o, lse, ws, scale=scale, stream=stream)
    return o, lse


def decode_chunk_workspace(q, k_cache):
    torch = _torch()
    B, Hq, Nq, d = q.shape
    _, Hkv, Nmax, _ = k_cache.shape
    return torch.empty(max(1, fa_decode_chunk_workspace_bytes(B, Hq, Hkv, Nq, Nmax, d)), dtype=torch.uint8,
                       device=q.device)


def decode_chunk(q, k_cache, v_cache, seqlens, causal=True, scale=None, workspace=None, stream=None):
    torch = _torch()
    B, Hq, Nq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    ws = decode_chunk_workspace(q, k_cache) if workspace is None else workspace
    fa_decode_chunk(q, k_cache, v_cache, seqlens, o, lse, ws, causal=causal, scale=scale, stream=stream)
    return o, lse


def decode_paged(q, k_pages, v_pages, block_table, seqlens, causal=True, scale=None, workspace=None, stream=None):
    torch = _torch()
    B, Hq, Nq, d = q.shape
    Hkv = k_pages.shape[1]
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(1, fa_decode_paged_workspace_bytes(B, Hq, Hkv, Nq, d)), dtype=torch.uint8,
                                device=q.device)
    fa_decode_paged(q, k_pages, v_pages, block_table, seqlens, o, lse, workspace, causal=causal, scale=scale,
                    stream=stream)
    return o, lse


def fwd_fp8(q8, k8, v8, descale_q, descale_k, descale_v, causal=False, scale=None, stream=None):
    torch = _torch()
    B, Hq, Nq, d = q8.shape
    o = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q8.device)
    fa_fwd_fp8(q8, k8, v8, o, lse, descale_q, descale_k, descale_v, causal=causal, scale=scale, stream=stream)
    return o, lse
