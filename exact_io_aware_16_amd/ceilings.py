"""Binding of libfa_ceilings (``include/fa_ceilings.h``): measured ceilings of
the GPU the attention kernels run on, for the benchmark to report beside the
published peaks.  Argument marshalling and timing with HIP events on the
launch stream only; every measurement runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa_ceilings.so")

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa_ceilings.so once (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_io_aware_16_amd.build`")
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    ip = ctypes.POINTER(ctypes.c_int)
    lib.fa_ceil_device.restype = i
    lib.fa_ceil_device.argtypes = [ip, ip, ip]
    lib.fa_ceil_mfma_bf16.restype = i
    lib.fa_ceil_mfma_bf16.argtypes = [vp, vp, i, i, vp]
    lib.fa_ceil_hbm_read.restype = i
    lib.fa_ceil_hbm_read.argtypes = [vp, sz, vp, i, i, vp]
    lib.fa_ceil_lds_read.restype = i
    lib.fa_ceil_lds_read.argtypes = [vp, vp, i, i, i, vp]
    lib.fa_ceil_hbm_read_lds_bytes.restype = ctypes.c_longlong
    lib.fa_ceil_hbm_read_lds_bytes.argtypes = [sz, i, i]
    lib.fa_ceil_hbm_read_lds.restype = i
    lib.fa_ceil_hbm_read_lds.argtypes = [vp, sz, i, i, i, i, vp]
    _lib = lib
    return lib


def _ok(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with HIP error {rc}")


def device():
    """(compute units, wall-tick rate in Hz, peak core clock in Hz)."""
    lib = load_library()
    n, w, p = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _ok(lib.fa_ceil_device(ctypes.byref(n), ctypes.byref(w), ctypes.byref(p)), "fa_ceil_device")
    return n.value, w.value * 1e3, p.value * 1e3


def _timed(launch, reps):
    """Per-launch seconds (HIP events on torch's current stream) of `reps` launches."""
    import torch
    st = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    en = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for a, b in zip(st, en):
        a.record()
        launch()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e-3 for a, b in zip(st, en)]


def _clock(stamps, wall_hz):
    """Median over waves of core cycles per wall second, and the median core
    cycles each wave spent in its loop."""
    import numpy as np
    s = stamps.cpu().numpy().astype(np.float64).reshape(-1, 4)
    dc, dw = s[:, 1] - s[:, 0], s[:, 3] - s[:, 2]
    ok = dw > 0
    return float(np.median(dc[ok] / dw[ok]) * wall_hz), float(np.median(dc))


def mfma_bf16(waves_per_simd=2, iters=20000, reps=5):
    """bf16 matrix-core throughput (FLOP/s) with `waves_per_simd` waves on every
    SIMD of every CU, the core clock those waves saw (Hz), and the core cycles
    per v_mfma_f32_32x32x16_bf16 per SIMD."""
    import numpy as np
    import torch
    lib = load_library()
    ncu, wall_hz, _ = device()
    wgs = ncu * waves_per_simd
    sink = torch.empty(wgs * 4, dtype=torch.float32, device="cuda:0")
    stamps = torch.empty(wgs * 16, dtype=torch.int64, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    launch = lambda: _ok(lib.fa_ceil_mfma_bf16(ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stamps.data_ptr()),
                                               wgs, iters, stream), "fa_ceil_mfma_bf16")
    launch()
    ts = _timed(launch, reps)
    flops = wgs * 4 * 4 * 32768.0 * iters
    t = float(np.median(ts))
    clk, cyc = _clock(stamps, wall_hz)
    return {"flops_per_s": flops / t, "clock_hz": clk,
            "cycles_per_mfma_per_simd": cyc / (4 * iters * waves_per_simd), "seconds": t}


def hbm_read(nbytes=4 << 30, wgs_per_cu=8, loads_in_flight=8, reps=10):
    """Streaming-read bandwidth (bytes/s) over an nbytes device buffer."""
    import numpy as np
    import torch
    lib = load_library()
    ncu, _, _ = device()
    wgs = ncu * wgs_per_cu
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
    sink = torch.empty(wgs * 256 * 16, dtype=torch.uint8, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    launch = lambda: _ok(lib.fa_ceil_hbm_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                              wgs, loads_in_flight, stream), "fa_ceil_hbm_read")
    launch()
    ts = _timed(launch, reps)
    del buf
    torch.cuda.empty_cache()
    return {"bytes_per_s": nbytes / float(np.median(ts)), "bytes": nbytes, "workgroups": wgs,
            "loads_in_flight": loads_in_flight}


def hbm_read_lds(nbytes=4 << 30, waves_per_cu=4, stage_kb=16, stages=3, nontemporal=True, reps=10):
    """Streaming-read bandwidth (bytes/s) through direct-to-LDS loads, one-wave
    workgroups with a private ring of `stages` stages of `stage_kb` KB."""
    import numpy as np
    import torch
    lib = load_library()
    ncu, _, _ = device()
    wgs = ncu * waves_per_cu
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
    nread = lib.fa_ceil_hbm_read_lds_bytes(nbytes, wgs, stage_kb)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    launch = lambda: _ok(lib.fa_ceil_hbm_read_lds(ctypes.c_void_p(buf.data_ptr()), nbytes, wgs, stage_kb, stages,
                                                  1 if nontemporal else 0, stream), "fa_ceil_hbm_read_lds")
    launch()
    ts = _timed(launch, reps)
    del buf
    torch.cuda.empty_cache()
    return {"bytes_per_s": nread / float(np.median(ts)), "bytes": nread, "workgroups": wgs, "stage_kb": stage_kb,
            "stages": stages, "nontemporal": bool(nontemporal)}


def lds_read(mode, clock_hz, wgs_per_cu=2, iters=4000, reps=3):
    """LDS read rate with 4 * wgs_per_cu waves on every CU: mode 0
    ds_read_b128, mode 1 ds_read_b64_tr_b16 (swizzled tile), mode 2
    ds_read_b64, mode 3 ds_read_b64_tr_b16 (unswizzled tile).  Bytes per
    second from the launch time (HIP events), and per core cycle per CU at
    clock_hz (the clock measured under matrix-core load)."""
    import numpy as np
    import torch
    lib = load_library()
    ncu, _, _ = device()
    wgs = ncu * wgs_per_cu
    sink = torch.empty(wgs * 256, dtype=torch.int32, device="cuda:0")
    stamps = torch.empty(wgs * 16, dtype=torch.int64, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    launch = lambda: _ok(lib.fa_ceil_lds_read(ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stamps.data_ptr()),
                                              mode, wgs, iters, stream), "fa_ceil_lds_read")
    launch()
    ts = _timed(launch, reps)
    per_read = 1024 if mode == 0 else 512
    rate = wgs * 4 * iters * 4 * per_read / float(np.median(ts))
    return {"bytes_per_s": rate, "bytes_per_clk_per_cu": rate / ncu / clock_hz}
