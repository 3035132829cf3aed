"""Shared helpers for the GPU parity tests (not a test module).

Inputs come from ``workloads`` (host, seeded); they are uploaded bit for bit.
Expected values come only from ``oracle``.
"""
import sys

import numpy as np

import oracle

TOL_BF16 = {"max_abs": 2e-2, "rel_l2": 5e-3}
TOL_F32 = {"max_abs": 1e-5}


def torch_mod():
    import torch
    return torch


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def to_device(arr):
    """uint16 bf16 bits -> torch.bfloat16 on cuda:0; float32 -> float32; int32 -> int32."""
    torch = torch_mod()
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(np.ascontiguousarray(arr)).to("cuda:0")


def to_host(t):
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def assert_close(name, gpu, ref, tol):
    m = oracle.compare(gpu, ref)
    print(f"  {name}: max_abs={m['max_abs']:.3e} rel_l2={m.get('rel_l2', 0):.3e}", flush=True)
    assert not m.get("nonfinite_mismatch"), f"{name}: non-finite pattern differs"
    assert m["max_abs"] <= tol["max_abs"], (name, m)
    if "rel_l2" in tol:
        assert m["rel_l2"] <= tol["rel_l2"], (name, m)


def announce(msg):
    print(msg, flush=True)
    sys.stdout.flush()
