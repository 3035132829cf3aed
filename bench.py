#!/usr/bin/env python3
"""Benchmark of libfa on one MI355X: exact causal attention forward/backward
TFLOP/s against the bf16 matrix-core peak, and KV-cache decode GB/s against HBM.

Prints ONE JSON line.  The headline ``value`` is the causal forward of the
B4 H16 N2048 d64 bf16 workload (TFLOP/s, algorithmic FLOPs 4*B*H*d*N(N+1)/2).
The same line carries every other measured row of the hot path:
``rows.fwd_llama`` (B2 H32 N8192 d128 causal forward), ``rows.fwd_bwd``
(B2 H16 N4096 d128 causal forward + backward, backward FLOPs counted as the five
products 10*B*H*d*pairs), and ``rows.decode`` (B16 Hq32 Hkv8 d128 GQA decode
over a 32768-slot cache with seeded lengths in [4096, 32768], bytes = the valid
K and V rows read once; the cache-cold number empties the 256 MB Infinity Cache
by reading a 1 GiB buffer between iterations).

Inputs are seeded synthetic tensors already resident in HBM when timing
starts.  Times come from HIP events recorded on the stream the kernels are
launched on (torch's current stream): a step is one call of the library, K
steps run back to back between one pair of events (arguments marshalled once,
so the host keeps the GPU fed), synchronised on both sides.  Each timed
section first runs its own step untimed for ``--settle`` seconds (default 0.3)
and then W warmup steps: the GPU raises its clock over the first tens of
milliseconds of sustained load, and timing inside that ramp (after host-side
set-up left the GPU idle) under-reports a 45 us kernel by up to 20%.  The headline also
reports the same launches timed one at a time ("isolated_launch"), where the
GPU idles between launches.  Decode's cache-cold figures need a cache-emptying
pass before every launch, so they are timed one launch at a time.

``cpu_baseline`` times the fp64 CPU oracle (materialising S and P) on a bounded
sample of the headline workload on this host's cores and checks the GPU output
of the same heads against it.  It is context, not a competitor.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal attn fwd/bwd TFLOP/s and % MFMA peak; decode HBM GB/s"
PEAK_BF16 = 2.5e15          # MI355X dense bf16 matrix-core peak, FLOP/s
PEAK_HBM = 8.0e12           # MI355X HBM3E bandwidth, bytes/s
PEAK_FP8 = 5.0e15           # MI355X dense fp8 matrix-core peak, FLOP/s
PROFILES = os.path.join(ROOT, "profiles")


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--headline-only", action="store_true", help="skip the other rows and the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU budget of the oracle sample")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed load before each timed section, so the GPU clock has ramped up")
    ap.add_argument("--only", choices=["fwd_llama", "fwd_fp8", "fwd_bwd", "fwd_bwd_gqa", "decode", "decode_chunk",
                                       "decode_paged"],
                    default=None,
                    help="run only this row (for profiling one kernel); prints the row as JSON")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run 3 plain 256 MiB device copies (known bytes) to scale rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE counts")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# timing helpers (HIP events on the launch stream)
# ---------------------------------------------------------------------------

SETTLE_S = 0.3   # seconds of untimed load before each timed section (--settle)


def settle(fn, before=None):
    """Run the step untimed, in batches of 16 with a synchronisation after each,
    for SETTLE_S seconds of wall time.  The GPU raises its clock over the first
    tens of milliseconds of sustained load (a d=64 forward runs 54 us per
    launch at first and 45 us after ~60 ms), and every section below is timed
    after host-side set-up during which the GPU idled, so without this the first
    few milliseconds of each section measure the ramp rather than the kernel."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(16):
            if before:
                before()
            fn()
        torch.cuda.synchronize()


def time_steps(fn, steps, warmup):
    """K back-to-back steps between one pair of HIP events on the launch stream
    (torch's current stream), synchronised on both sides, after the clock
    settle and W warmup steps; returns seconds per step and the host wall time
    of the timed region."""
    import torch
    settle(fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) * 1e-3 / steps, wall


def time_launches(fn, steps, warmup, before=None):
    """Per-launch event pairs (after the clock settle and W warmup launches);
    returns (list of seconds, total seconds of the timed region)."""
    import torch
    settle(fn, before)
    for _ in range(warmup):
        if before:
            before()
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        if before:
            before()
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [s.elapsed_time(e) * 1e-3 for s, e in zip(starts, ends)], wall


def stats(ts):
    import numpy as np
    a = np.sort(np.asarray(ts))
    return {"median_us": float(np.median(a) * 1e6), "min_us": float(a[0] * 1e6),
            "p90_us": float(a[int(0.9 * (len(a) - 1))] * 1e6), "mean_us": float(a.mean() * 1e6)}


def causal_pairs(Nq, Nk):
    # pairs (i, j) with j <= i + Nk - Nq
    off = Nk - Nq
    return sum(min(Nk, i + off + 1) for i in range(Nq))


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


FWD_SOURCES = ["exact_io_aware_16_amd/csrc/fa_fwd.hip", "exact_io_aware_16_amd/csrc/fa_device.h"]


def measured_traffic(name, digest, launches_per_run=1):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE counts,
    only if they were taken on the current kernel source (else None)."""
    path = os.path.join(PROFILES, f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != digest:
        return None
    return float(t["hbm_bytes_per_launch"])


# ---------------------------------------------------------------------------
# the rows
# ---------------------------------------------------------------------------

def upload(w):
    import numpy as np
    import torch
    out = {}
    for n, a in w.tensors.items():
        if a.dtype == np.uint16:
            out[n] = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
        else:
            out[n] = torch.from_numpy(a).to("cuda:0")
    return out


def headline(args, fa, W):
    import torch
    w = W.make_config(2)
    t = upload(w)
    q, k, v = t["q"], t["k"], t["v"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda:0")
    run = fa.prepare_fwd(q, k, v, o, lse, causal=True, scale=w.scale)
    avg, wall = time_steps(run, args.steps, args.warmup)
    # the same launches one at a time (each between its own events), for spread
    ts, _ = time_launches(run, max(10, args.steps // 5), 2)
    flops = 4.0 * w.B * w.Hq * w.d * causal_pairs(w.Nq, w.Nk)
    st = {"per_step_us": avg * 1e6, "isolated_launch": stats(ts)}
    algo_bytes = 2 * (w.B * w.Hq * w.Nq * w.d * 2) + 2 * (w.B * w.Hkv * w.Nk * w.d * 2) + w.B * w.Hq * w.Nq * 4
    digest = source_digest(FWD_SOURCES)
    traffic = measured_traffic("fwd_bf16_causal_d64_B4H16N2048", digest)
    return {
        "w": w, "tensors": t, "out": (o, lse), "flops": flops, "avg_s": avg, "stats": st, "wall": wall,
        "roofline": {"bound": "mfma", "achieved": flops / avg / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                     "frac": flops / avg / PEAK_BF16, "traffic": traffic,
                     "kernel": "fa::fwd_ring_kernel<64, 4, 2, 1, true>", "flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": algo_bytes, "avg_launch_us": avg * 1e6,
                     "source_digest": digest},
    }


def row_fwd_llama(args, fa, W):
    import torch
    w = W.make_config(3)
    t = upload(w)
    o = torch.empty_like(t["q"])
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda:0")
    run = fa.prepare_fwd(t["q"], t["k"], t["v"], o, lse, causal=True, scale=w.scale)
    avg, _ = time_steps(run, max(5, args.steps // 5), max(2, args.warmup // 2))
    flops = 4.0 * w.B * w.Hq * w.d * causal_pairs(w.Nq, w.Nk)
    return {"workload": w.name, "tflops": flops / avg / 1e12, "frac_of_peak": flops / avg / PEAK_BF16,
            "flops_per_launch": flops, "per_step_us": avg * 1e6}


def row_fwd_fp8(args, fa, W):
    """The LLaMA-shaped causal forward with E4M3 inputs (per-tensor descales)."""
    import torch
    w = W.make_config(3)
    f8 = W.to_fp8(w)
    dev = {n: torch.from_numpy(c).to("cuda:0") for n, (c, _) in f8.items()}
    o = torch.empty((w.B, w.Hq, w.Nq, w.d), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda:0")
    run = fa.prepare_fwd_fp8(dev["q"], dev["k"], dev["v"], o, lse, f8["q"][1], f8["k"][1], f8["v"][1], causal=True,
                             scale=w.scale)
    avg, _ = time_steps(run, max(5, args.steps // 5), max(2, args.warmup // 2))
    flops = 4.0 * w.B * w.Hq * w.d * causal_pairs(w.Nq, w.Nk)
    return {"workload": "llama_causal_fwd_B2_H32_N8192_d128_fp8_e4m3_kout", "tflops": flops / avg / 1e12,
            "frac_of_fp8_peak": flops / avg / PEAK_FP8, "flops_per_launch": flops, "per_step_us": avg * 1e6}


def row_fwd_bwd(args, fa, W, **override):
    import torch
    w = W.make_config(5, **override)
    t = upload(w)
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda:0")
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda:0")
    dk = torch.empty(k.shape, dtype=torch.float32, device="cuda:0")
    dv = torch.empty(v.shape, dtype=torch.float32, device="cuda:0")
    ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.Hq, w.Nq, w.d), dtype=torch.uint8, device="cuda:0")
    n = max(5, args.steps // 5)
    af, _ = time_steps(fa.prepare_fwd(q, k, v, o, lse, causal=True, scale=w.scale), n, 3)
    ab, _ = time_steps(fa.prepare_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal=True, scale=w.scale), n, 3)
    pairs = causal_pairs(w.Nq, w.Nk)
    ff = 4.0 * w.B * w.Hq * w.d * pairs
    fb = 10.0 * w.B * w.Hq * w.d * pairs
    name = w.name if not override else f"causal_fwd_bwd_B{w.B}_Hq{w.Hq}_Hkv{w.Hkv}_N{w.Nq}_d{w.d}_bf16"
    return {"workload": name, "fwd_tflops": ff / af / 1e12, "fwd_frac_of_peak": ff / af / PEAK_BF16,
            "bwd_tflops": fb / ab / 1e12, "bwd_frac_of_peak": fb / ab / PEAK_BF16,
            "bwd_flop_convention": "10*B*H*d*pairs (five products, recompute included)",
            "fwd_bwd_tflops": (ff + fb) / (af + ab) / 1e12, "fwd_per_step_us": af * 1e6,
            "bwd_per_step_us": ab * 1e6}


def row_decode(args, fa, W):
    import numpy as np
    import torch
    w = W.make_config(4)
    t = upload(w)
    sl = torch.from_numpy(w.seqlens).to("cuda:0")
    q, k, v = t["q"], t["k"], t["v"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda:0")
    ws = fa.decode_workspace(q, k)
    run = fa.prepare_decode(q, k, v, sl, o, lse, ws, scale=w.scale)
    valid = int(w.seqlens.astype(np.int64).sum())
    nbytes = valid * w.Hkv * w.d * 2 * 2 + q.numel() * 2 + o.numel() * 2 + lse.numel() * 4
    n = max(10, args.steps // 2)
    aw, _ = time_steps(run, n, 5)
    # 1 GiB (> the 256 MB Infinity Cache + L2s) to push the cache out between launches
    flush = torch.zeros(1 << 28, dtype=torch.float32, device="cuda:0")
    flush.sum()
    torch.cuda.synchronize()
    # by reading it: the caches then hold only clean lines of the flush buffer
    tc, _ = time_launches(run, n, 2, before=lambda: flush.sum())
    # by writing it: the launch also pays for evicting up to 256 MB of dirty lines
    td, _ = time_launches(run, n, 2, before=lambda: flush.fill_(1.0))
    sc, sd = stats(tc), stats(td)
    gbps = lambda st: nbytes / (st["median_us"] * 1e-6) / 1e9
    warm = nbytes / aw / 1e9
    return {"workload": w.name, "valid_keys": valid, "algorithmic_bytes": nbytes,
            "cold_gbps": gbps(sc), "cold_frac_of_hbm": gbps(sc) * 1e9 / PEAK_HBM,
            "warm_gbps": warm, "warm_frac_of_hbm": warm * 1e9 / PEAK_HBM,
            "cold_after_writes_gbps": gbps(sd),
            "cold": sc, "warm_per_step_us": aw * 1e6, "cold_after_writes": sd,
            "note": "graded: cold = caches emptied (by reading a 1 GiB buffer) before each launch; "
                    "warm = back-to-back launches; cold_after_writes = caches filled with dirty lines first"}


def row_decode_chunk(args, fa, W):
    """Chunk decode on the decode workload's cache: 8 new tokens per head
    (causal to each sequence's length), as when a large model checks 8 drafted
    tokens; bytes as decode (valid K/V once) plus the larger q, o and lse."""
    import numpy as np
    import torch
    nq = 8
    w = W.make_config(4, Nq=nq)
    t = upload(w)
    sl = torch.from_numpy(w.seqlens).to("cuda:0")
    q, k, v = t["q"], t["k"], t["v"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, nq), dtype=torch.float32, device="cuda:0")
    ws = fa.decode_chunk_workspace(q, k)
    run = fa.prepare_decode_chunk(q, k, v, sl, o, lse, ws, causal=True, scale=w.scale)
    valid = int(w.seqlens.astype(np.int64).sum())
    nbytes = valid * w.Hkv * w.d * 2 * 2 + q.numel() * 2 + o.numel() * 2 + lse.numel() * 4
    flops = 4 * w.Hq * w.d * sum(int(n) * nq - nq * (nq - 1) // 2 for n in w.seqlens)
    n = max(10, args.steps // 2)
    flush = torch.zeros(1 << 28, dtype=torch.float32, device="cuda:0")
    flush.sum()
    torch.cuda.synchronize()
    tc, _ = time_launches(run, n, 2, before=lambda: flush.sum())
    sc = stats(tc)
    gbps = nbytes / (sc["median_us"] * 1e-6) / 1e9
    return {"workload": "gqa_decode_chunk_B16_Hq32_Hkv8_Nq8_N32768_d128_bf16_causal", "valid_keys": valid,
            "algorithmic_bytes": nbytes, "cold_gbps": gbps, "cold_frac_of_hbm": gbps * 1e9 / PEAK_HBM,
            "tflops": flops / (sc["median_us"] * 1e-6) / 1e12, "cold": sc,
            "note": "caches emptied (by reading a 1 GiB buffer) before each launch"}


def row_decode_paged(args, fa, W):
    """The decode workload with its cache in 64-key pages at seeded random
    positions of a page pool, reached through a block table."""
    import numpy as np
    import torch
    P = 64
    w = W.make_config(4)
    t = upload(w)
    sl = torch.from_numpy(w.seqlens).to("cuda:0")
    q = t["q"]
    mp = w.Nk // P
    perm = torch.from_numpy(np.random.Generator(np.random.PCG64(4)).permutation(w.B * mp).astype(np.int64)).to("cuda:0")

    def paged(x):   # [B, Hkv, mp*P, d] -> pool [B*mp, Hkv, P, d], page (b, p) at perm[b*mp + p]
        pool = torch.empty((w.B * mp, w.Hkv, P, w.d), dtype=x.dtype, device="cuda:0")
        pool[perm] = x.view(w.B, w.Hkv, mp, P, w.d).permute(0, 2, 1, 3, 4).reshape(w.B * mp, w.Hkv, P, w.d)
        return pool
    kp, vp = paged(t["k"]), paged(t["v"])
    del t
    table = perm.view(w.B, mp).to(torch.int32).contiguous()
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, 1), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(max(1, fa.fa_decode_paged_workspace_bytes(w.B, w.Hq, w.Hkv, 1, w.d)), dtype=torch.uint8,
                     device="cuda:0")
    run = fa.prepare_decode_paged(q, kp, vp, table, sl, o, lse, ws, causal=True, scale=w.scale)
    valid = int(w.seqlens.astype(np.int64).sum())
    nbytes = valid * w.Hkv * w.d * 2 * 2 + q.numel() * 2 + o.numel() * 2 + lse.numel() * 4
    n = max(10, args.steps // 2)
    flush = torch.zeros(1 << 28, dtype=torch.float32, device="cuda:0")
    flush.sum()
    torch.cuda.synchronize()
    tc, _ = time_launches(run, n, 2, before=lambda: flush.sum())
    sc = stats(tc)
    gbps = nbytes / (sc["median_us"] * 1e-6) / 1e9
    return {"workload": "gqa_decode_paged_B16_Hq32_Hkv8_N32768_d128_bf16_page64", "valid_keys": valid,
            "algorithmic_bytes": nbytes, "cold_gbps": gbps, "cold_frac_of_hbm": gbps * 1e9 / PEAK_HBM,
            "cold": sc, "note": "64-key pages at seeded random pool positions; caches emptied (by reading a "
                                "1 GiB buffer) before each launch"}


def cpu_baseline(args, head, W):
    """The fp64 oracle on the host cores, on whole heads of the headline workload,
    until the CPU budget is spent; also checks the GPU's output on those heads."""
    import numpy as np
    import oracle
    w = head["w"]
    o_gpu = head["out"][0].float().cpu().numpy()
    l_gpu = head["out"][1].cpu().numpy()
    q, k, v = w.values("q"), w.values("k"), w.values("v")
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    done, t_cpu = [], 0.0
    worst = {"max_abs": 0.0, "rel_l2": 0.0}
    for b, h in heads:
        t0 = time.perf_counter()
        O, L = oracle.ref_fwd(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], causal=True,
                              scale=w.scale)
        t_cpu += time.perf_counter() - t0
        done.append((b, h))
        for name, g, r in (("O", o_gpu[b, h], O[0, 0]), ("LSE", l_gpu[b, h], L[0, 0])):
            m = oracle.compare(g, r)
            worst["max_abs"] = max(worst["max_abs"], m["max_abs"])
            worst["rel_l2"] = max(worst["rel_l2"], m["rel_l2"])
        if t_cpu >= args.cpu_seconds:
            break
    flops = 4.0 * len(done) * w.d * causal_pairs(w.Nq, w.Nk)
    return {"value": flops / t_cpu / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(done)} of {len(heads)} (batch, head) slices of the headline workload "
                      f"(N={w.Nq}, d={w.d}, causal), fp64 numpy materialising S and P; "
                      f"rate = causal algorithmic FLOPs / oracle seconds",
            "seconds": t_cpu, "gpu_vs_oracle_on_sample": worst,
            "gpu_speedup_vs_oracle": (head["flops"] / head["avg_s"]) / (flops / t_cpu)}


def main():
    global SETTLE_S
    args = parse_args()
    SETTLE_S = max(0.0, args.settle)
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); the multi-GPU path is not built. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py is single-process; WORLD_SIZE > 1 is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    import exact_io_aware_16_amd as fa
    import workloads as W
    fa.load_library()   # raises if libfa.so is not built: there is no other path

    if args.only:
        fn = {"fwd_llama": row_fwd_llama, "fwd_bwd": row_fwd_bwd, "decode": row_decode,
              "fwd_bwd_gqa": lambda a, f, w_: row_fwd_bwd(a, f, w_, Hq=32, Hkv=8), "fwd_fp8": row_fwd_fp8,
              "decode_chunk": row_decode_chunk, "decode_paged": row_decode_paged}[args.only]
        print(json.dumps({args.only: fn(args, fa, W)}), flush=True)
        return

    log("headline: causal forward B4 H16 N2048 d64 bf16")
    head = headline(args, fa, W)
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    rows = {}
    if not args.headline_only:
        log("row: causal forward B2 H32 N8192 d128 bf16")
        rows["fwd_llama"] = row_fwd_llama(args, fa, W)
        torch.cuda.empty_cache()
        log("row: causal forward B2 H32 N8192 d128 fp8 (E4M3)")
        rows["fwd_fp8"] = row_fwd_fp8(args, fa, W)
        torch.cuda.empty_cache()
        log("row: causal forward + backward B2 H16 N4096 d128 bf16")
        rows["fwd_bwd"] = row_fwd_bwd(args, fa, W)
        torch.cuda.empty_cache()
        log("row: GQA causal forward + backward B2 Hq32 Hkv8 N4096 d128 bf16")
        rows["fwd_bwd_gqa"] = row_fwd_bwd(args, fa, W, Hq=32, Hkv=8)
        torch.cuda.empty_cache()
        log("row: GQA decode B16 Hq32 Hkv8 N32768 d128 bf16")
        rows["decode"] = row_decode(args, fa, W)
        torch.cuda.empty_cache()
        log("row: GQA chunk decode B16 Hq32 Hkv8 Nq8 N32768 d128 bf16")
        rows["decode_chunk"] = row_decode_chunk(args, fa, W)
        torch.cuda.empty_cache()
        log("row: GQA decode against a paged cache (64-key pages) B16 Hq32 Hkv8 N32768 d128 bf16")
        rows["decode_paged"] = row_decode_paged(args, fa, W)
        torch.cuda.empty_cache()
    cpu = None
    if not args.headline_only and not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle on a sample of the headline workload")
        cpu = cpu_baseline(args, head, W)

    w = head["w"]
    line = {
        "metric": METRIC,
        "value": head["flops"] / head["avg_s"] / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["avg_s"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16 round-to-nearest-even)",
        "config": {"workload": w.name, "B": w.B, "H": w.Hq, "N": w.Nq, "d": w.d, "causal": True,
                   "flops_per_step": head["flops"], "flop_convention": "4*B*H*d*N(N+1)/2"},
        "frac_of_peak": head["flops"] / head["avg_s"] / PEAK_BF16,
        "timing": head["stats"],
        "clock_settle_s": SETTLE_S,
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "rows": rows,
        "context": {"pages_claims": "2-4x faster and 10-20x less memory than standard attention; "
                                    "FlashAttention-3 1.5-2 PFLOP/s on NVIDIA H100 (other hardware, not a target)"},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
