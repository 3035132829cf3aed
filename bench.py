#!/usr/bin/env python3
"""Benchmark of libfa on one MI355X: exact causal attention forward/backward
TFLOP/s against the bf16 matrix-core peak, and KV-cache decode GB/s against HBM.

Prints ONE JSON line.  The headline ``value`` is the causal forward of the
LLaMA-shaped workload, B2 H32 N8192 d128 bf16 with 1% of the key rows scaled
by 8 (TFLOP/s, algorithmic FLOPs 4*B*H*d*N(N+1)/2): the largest configuration
of the metric that fits one GPU.  ``roofline`` is that kernel's; ``cpu_baseline``
times the fp64 CPU oracle on sampled query rows of the same workload.  The
same line carries every other row of the hot path, each with its own timing
spread (median/min/p90 of per-launch HIP events), roofline block and parity
against the oracle:
``rows.fwd_small`` (B1 H1 N256 d64 fp32, non-causal), ``rows.fwd_causal_d64``
(B4 H16 N2048 d64 causal), ``rows.fwd_fp8`` (the headline workload in FP8
E4M3), ``rows.fwd_bwd`` (B2 H16 N4096 d128 causal forward + backward, backward
FLOPs counted as the five products 10*B*H*d*pairs), ``rows.fwd_bwd_gqa``
(the same at Hq32 Hkv8), ``rows.decode`` (B16 Hq32 Hkv8 d128 GQA decode over a
32768-slot cache with seeded lengths in [4096, 32768], bytes = the valid K and
V rows read once; the graded number empties the 256 MB Infinity Cache before
each launch), ``rows.decode_chunk`` and ``rows.decode_paged``.
``measured_ceilings`` reports what this part delivers to a kernel at all:
bf16 matrix-core throughput and the clock it runs at, streaming HBM read
bandwidth, LDS read rates.

Inputs are seeded synthetic tensors already resident in HBM when timing
starts.  Times come from HIP events recorded on the stream the kernels are
launched on (torch's current stream): a step is one call of the library, K
steps run back to back between one pair of events (arguments marshalled once,
so the host keeps the GPU fed), synchronised on both sides.  Each timed
section first runs its own step untimed for ``--settle`` seconds (default 0.3)
and then W warmup steps: the GPU raises its clock over the first tens of
milliseconds of sustained load, and timing inside that ramp (after host-side
set-up left the GPU idle) under-reports a short kernel by up to 20%.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only]
"""
from __future__ import annotations

import os

# The CPU baseline's numpy runs on every host core this process may use; the
# thread count is fixed here, before numpy (or torch, which imports it) loads.
_HOST_CORES = len(os.sched_getaffinity(0))
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_var, str(_HOST_CORES))

import argparse  # noqa: E402
import hashlib  # noqa: E402
import json  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal attn fwd/bwd TFLOP/s and % MFMA peak; decode HBM GB/s"
PEAK_BF16 = 2.5e15          # MI355X dense bf16 matrix-core peak, FLOP/s (at 2.4 GHz)
PEAK_HBM = 8.0e12           # MI355X HBM3E bandwidth, bytes/s
PEAK_FP8 = 5.0e15           # MI355X dense fp8 matrix-core peak, FLOP/s
PEAK_FP32_VALU = 157.3e12   # MI355X fp32 vector peak, FLOP/s
PROFILES = os.path.join(ROOT, "profiles")
SETTLE_S = 0.3              # seconds of untimed load before each timed section (--settle)

FWD_SOURCES = ["exact_io_aware_16_amd/csrc/fa_fwd.hip", "exact_io_aware_16_amd/csrc/fa_device.h"]
FP8_SOURCES = ["exact_io_aware_16_amd/csrc/fa_fwd_fp8.hip", "exact_io_aware_16_amd/csrc/fa_device.h"]
BWD_SOURCES = ["exact_io_aware_16_amd/csrc/fa_bwd.hip", "exact_io_aware_16_amd/csrc/fa_device.h"]
DEC_SOURCES = ["exact_io_aware_16_amd/csrc/fa_decode.hip", "exact_io_aware_16_amd/csrc/fa_device.h"]

ROWS = ["fwd_small", "fwd_causal_d64", "fwd_fp8", "fwd_bwd", "fwd_bwd_gqa", "decode", "decode_chunk",
        "decode_paged"]

# Kernels of the three traffic summaries (per call: each launched once).
HEAD_KERNEL = "fa::fwd_ring_kernel<128, 8, 2, 1, true>"
BWD_KERNELS = ["fa::bwd_dq_kernel<128, true, float>", "fa::bwd_dkdv_kernel<128, true, float>"]
DEC_KERNELS = ["fa::decode_stream_kernel<128, 3, 4>", "fa::decode_stream_combine_kernel<128>"]
CHUNK_KERNELS = ["fa::decode_stream_kernel<128, 2, 32>", "fa::decode_stream_combine_kernel<128>"]
FP8_KERNEL = "fa::(anonymous namespace)::fwd_fp8_kernel<128, 4, 3, true>"


def _pmc_targets():
    """Per --pmc-target: the bench part to profile, the summary's name, the
    kernels counted per call, the sources whose digest the summary records,
    and the algorithmic bytes read and written per call."""
    # config 3: B2 H32 N8192 d128, causal forward (q, k, v bf16 in; o bf16, lse fp32 out)
    t3 = 2 * 32 * 8192
    # config 2: B4 H16 N2048 d64, causal forward
    t2 = 4 * 16 * 2048
    # config 5: B2 H16 N4096 d128 backward (q, k, v, o, dO bf16 and lse fp32 in; fp32 gradients out)
    t5 = 2 * 16 * 4096
    return {
        "headline": dict(only="headline", name="fwd_bf16_causal_d128_B2H32N8192", kernels=[HEAD_KERNEL],
                         sources=FWD_SOURCES, read=3 * t3 * 128 * 2, write=t3 * 128 * 2 + t3 * 4,
                         note="per launch of the causal forward"),
        "fwd_causal_d64": dict(only="fwd_causal_d64", name="fwd_bf16_causal_d64_B4H16N2048",
                               kernels=["fa::fwd_ring_kernel<64, 4, 2, 1, true>"], sources=FWD_SOURCES,
                               read=3 * t2 * 64 * 2, write=t2 * 64 * 2 + t2 * 4,
                               note="per launch of the causal forward"),
        "fwd_bwd": dict(only="fwd_bwd", name="bwd_bf16_causal_d128_B2H16N4096", kernels=BWD_KERNELS,
                        sources=BWD_SOURCES, read=5 * t5 * 128 * 2 + t5 * 4, write=3 * t5 * 128 * 4,
                        note="per fa_bwd call (dQ kernel + dK/dV kernel); the D and lse log2 e rows the dQ "
                             "kernel writes for the dK/dV kernel are counted in the measured bytes, not in "
                             "the algorithmic ones"),
        "fwd_bwd_gqa": dict(only="fwd_bwd_gqa", name="bwd_bf16_causal_gqa_d128_B2Hq32Hkv8N4096", kernels=BWD_KERNELS,
                            sources=BWD_SOURCES, read=3 * 2 * t5 * 128 * 2 + 2 * (t5 // 2) * 128 * 2 + 2 * t5 * 4,
                            write=2 * t5 * 128 * 4 + 2 * (t5 // 2) * 128 * 4,
                            note="per fa_bwd call (dQ kernel + dK/dV kernel) at B2 Hq32 Hkv8 N4096: q, o, dO and "
                                 "lse over 32 query heads, k and v over 8 K/V heads read; dq over 32 heads, dk and "
                                 "dv over 8 written (fp32)"),
        "fwd_fp8": dict(only="fwd_fp8", name="fwd_fp8_causal_d128_B2H32N8192", kernels=[FP8_KERNEL],
                        sources=FP8_SOURCES, read=3 * t3 * 128, write=t3 * 128 * 2 + t3 * 4,
                        note="per launch of the causal FP8 forward (E4M3 q, k, v in; bf16 o, fp32 lse out)"),
        "decode_chunk": dict(only="decode_chunk", name="decode_chunk_gqa_B16Hq32Hkv8_Nq8_N32768_d128",
                             kernels=CHUNK_KERNELS, sources=DEC_SOURCES, read=None, write=None,
                             note="per fa_decode_chunk call (stream kernel + combine), cache-cold launches"),
        "decode_paged": dict(only="decode_paged", name="decode_paged_gqa_B16Hq32Hkv8_N32768_d128_page64",
                             kernels=DEC_KERNELS, sources=DEC_SOURCES, read=None, write=None,
                             note="per fa_decode_paged call (stream kernel + combine), cache-cold launches"),
        "decode": dict(only="decode", name="decode_gqa_B16Hq32Hkv8_N32768_d128", kernels=DEC_KERNELS,
                       sources=DEC_SOURCES, read=None, write=None,
                       note="per fa_decode call (stream kernel + combine); the counted launches alternate "
                            "between the cache states of the bench row; writes include the float32 partial "
                            "results that the combine kernel reads back"),
    }


PMC_TARGETS = _pmc_targets()


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--headline-only", action="store_true", help="skip the other rows and the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured-ceiling kernels")
    ap.add_argument("--no-parity", action="store_true", help="skip the per-row oracle checks")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU budget of the oracle sample")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed load before each timed section, so the GPU clock has ramped up")
    ap.add_argument("--only", choices=["headline", "ceilings"] + ROWS, default=None,
                    help="run only this part (for profiling one kernel); prints it as JSON")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run 3 plain 256 MiB device copies (known bytes) to scale rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE counts")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="no GPU: turn the counter_collection.csv files of a FETCH_SIZE and a WRITE_SIZE "
                         "rocprofv3 pass (each run with --calibrate-copy) into profiles/<workload>_traffic.json")
    ap.add_argument("--pmc-target", choices=sorted(PMC_TARGETS), default="headline",
                    help="which kernels of the profiled run --pmc-summary reports")
    ap.add_argument("--pmc-out", default=None, help="where --pmc-summary writes (default profiles/)")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# timing helpers (HIP events on the launch stream)
# ---------------------------------------------------------------------------

def settle(fn, before=None):
    """Run the step untimed, in batches of 16 with a synchronisation after each,
    for SETTLE_S seconds of wall time, so the GPU clock has ramped up."""
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
    settle and W warmup steps; returns seconds per step."""
    import torch
    settle(fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e-3 / steps


def time_launches(fn, steps, warmup, before=None):
    """Per-launch event pairs (after the clock settle and W warmup launches)."""
    import torch
    settle(fn, before)
    for _ in range(warmup):
        if before:
            before()
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        if before:
            before()
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    return [s.elapsed_time(e) * 1e-3 for s, e in zip(starts, ends)]


def stats(ts):
    import numpy as np
    a = np.sort(np.asarray(ts))
    return {"median_us": float(np.median(a) * 1e6), "min_us": float(a[0] * 1e6),
            "p90_us": float(a[int(0.9 * (len(a) - 1))] * 1e6), "mean_us": float(a.mean() * 1e6), "launches": len(a)}


def measure(fn, steps, warmup):
    """Back-to-back mean (the rate) plus the per-launch spread."""
    avg = time_steps(fn, steps, warmup)
    spread = stats(time_launches(fn, max(10, steps // 2), 2))
    return avg, dict(per_step_us=avg * 1e6, **spread)


def causal_pairs(Nq, Nk):
    # pairs (i, j) with j <= i + Nk - Nq
    off = Nk - Nq
    return sum(max(0, min(Nk, i + off + 1)) for i in range(Nq))


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name, sources):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE counts,
    only if they were taken on the current kernel source (else None)."""
    path = os.path.join(PROFILES, f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != source_digest(sources):
        return None
    return float(t["hbm_bytes_per_launch"])


def roofline(bound, work, seconds, kernel, traffic_name=None, sources=None, peak=None, **extra):
    """The roofline block of one kernel: algorithmic work per launch over the
    measured launch time, against the part's published peak."""
    if bound == "mfma":
        peak, unit, scale = (peak or PEAK_BF16), "TFLOP/s", 1e12
    elif bound == "hbm":
        peak, unit, scale = PEAK_HBM, "GB/s", 1e9
    else:
        peak, unit, scale = (peak or PEAK_FP32_VALU), "TFLOP/s", 1e12
    traffic = measured_traffic(traffic_name, sources) if traffic_name else None
    out = {"bound": bound, "achieved": work / seconds / scale, "peak": peak / scale, "unit": unit,
           "frac": work / seconds / peak, "traffic": traffic, "kernel": kernel, "avg_launch_us": seconds * 1e6}
    if sources:
        out["source_digest"] = source_digest(sources)
    out.update(extra)
    return out


def parity(pairs, scope):
    """max-abs and rel-L2 of each (name, gpu, reference) against the oracle."""
    import oracle
    out = {"scope": scope}
    for name, g, r in pairs:
        m = oracle.compare(g, r)
        out[name] = {"max_abs": m["max_abs"], "rel_l2": m["rel_l2"]}
        if m.get("nonfinite_mismatch"):
            out[name]["nonfinite_mismatch"] = True
    return out


def host(t):
    import numpy as np
    return t.float().cpu().numpy().astype(np.float64)


def gather_rows(t, rows):
    """t[b, h, i] for each (b, h, i) of rows, on the host in float64."""
    import torch
    idx = torch.as_tensor(rows, dtype=torch.int64, device=t.device)
    return host(t[idx[:, 0], idx[:, 1], idx[:, 2]])


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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads():
    """Threads numpy's BLAS actually runs with (threadpoolctl), else the setting."""
    try:
        import threadpoolctl
        n = [p["num_threads"] for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return int(os.environ.get("OMP_NUM_THREADS", _HOST_CORES))


# ---------------------------------------------------------------------------
# measured ceilings
# ---------------------------------------------------------------------------

def ceilings():
    from exact_io_aware_16_amd import ceilings as C
    ncu, wall_hz, peak_clk = C.device()
    m1 = C.mfma_bf16(waves_per_simd=1)
    m2 = C.mfma_bf16(waves_per_simd=2)
    hbm = max((C.hbm_read(loads_in_flight=u, wgs_per_cu=g) for u in (4, 8, 16) for g in (4, 8)),
              key=lambda r: r["bytes_per_s"])
    hbm_lds = max((C.hbm_read_lds(waves_per_cu=w, stage_kb=16, stages=st, nontemporal=nt)
                   for nt in (True, False) for st in (2, 3) for w in (3, 4, 8)), key=lambda r: r["bytes_per_s"])
    clk = m1["clock_hz"]
    lds = {m: C.lds_read(m, clk) for m in (0, 1, 2, 3)}
    return {
        "compute_units": ncu, "peak_core_clock_ghz": peak_clk / 1e9,
        "mfma_bf16_tflops": max(m1["flops_per_s"], m2["flops_per_s"]) / 1e12,
        "mfma_bf16_frac_of_peak": max(m1["flops_per_s"], m2["flops_per_s"]) / PEAK_BF16,
        "mfma_bf16_tflops_one_wave_per_simd": m1["flops_per_s"] / 1e12,
        "mfma_bf16_tflops_two_waves_per_simd": m2["flops_per_s"] / 1e12,
        "core_clock_ghz_under_mfma": clk / 1e9,
        "hbm_read_gbps": hbm["bytes_per_s"] / 1e9,
        "hbm_read_frac_of_peak": hbm["bytes_per_s"] / PEAK_HBM,
        "hbm_read_config": {"workgroups": hbm["workgroups"], "loads_in_flight": hbm["loads_in_flight"]},
        "hbm_read_direct_to_lds_gbps": hbm_lds["bytes_per_s"] / 1e9,
        "hbm_read_direct_to_lds_frac_of_peak": hbm_lds["bytes_per_s"] / PEAK_HBM,
        "hbm_read_direct_to_lds_config": {k: hbm_lds[k] for k in ("workgroups", "stage_kb", "stages", "nontemporal")},
        "lds_read_b128_bytes_per_clk_per_cu": lds[0]["bytes_per_clk_per_cu"],
        "lds_read_tr_b16_bytes_per_clk_per_cu": lds[1]["bytes_per_clk_per_cu"],
        "lds_read_b64_bytes_per_clk_per_cu": lds[2]["bytes_per_clk_per_cu"],
        "lds_read_tr_b16_unswizzled_bytes_per_clk_per_cu": lds[3]["bytes_per_clk_per_cu"],
        "note": "fa_ceilings kernels: 4 independent v_mfma_f32_32x32x16_bf16 chains per wave on every SIMD "
                "(1 and 2 waves per SIMD); a 4 GiB non-temporal streaming read (best of 4/8/16 loads in flight per "
                "lane and 4/8 workgroups per CU); the same read through direct-to-LDS loads (one-wave workgroups, "
                "16 KB stages, best of 2/3 stages, 3/4/8 waves per CU, default or non-temporal policy); 64 KB of LDS re-read by 8 waves per CU (rates from launch time "
                "at the clock measured under MFMA load); clock = core-cycle counter over the constant-rate counter "
                "during the MFMA loop",
    }


# ---------------------------------------------------------------------------
# the rows
# ---------------------------------------------------------------------------

def fwd_workload(cfg):
    import torch
    import workloads as W
    w = W.make_config(cfg)
    t = upload(w)
    o = torch.empty_like(t["q"])
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda:0")
    return w, t, o, lse


def headline(args, fa):
    """Causal forward of the LLaMA-shaped workload (the metric's largest configuration)."""
    w, t, o, lse = fwd_workload(3)
    run = fa.prepare_fwd(t["q"], t["k"], t["v"], o, lse, causal=True, scale=w.scale)
    avg = time_steps(run, args.steps, args.warmup)
    spread = stats(time_launches(run, max(10, args.steps // 5), 2))
    flops = 4.0 * w.B * w.Hq * w.d * causal_pairs(w.Nq, w.Nk)
    algo_bytes = 2 * (w.B * w.Hq * w.Nq * w.d * 2) + 2 * (w.B * w.Hkv * w.Nk * w.d * 2) + w.B * w.Hq * w.Nq * 4
    return {
        "w": w, "out": (o, lse), "flops": flops, "avg_s": avg,
        "timing": dict(per_step_us=avg * 1e6, **spread),
        "roofline": roofline("mfma", flops, avg, HEAD_KERNEL,
                             "fwd_bf16_causal_d128_B2H32N8192", FWD_SOURCES, flops_per_launch=flops,
                             algorithmic_bytes_per_launch=algo_bytes),
    }


def cpu_baseline(args, head):
    """The fp64 oracle (ref_fwd_rows: each sampled query row against its own
    keys, S and P materialised) on this host's cores: the 512 parity rows of the
    headline workload, then further seeded rows until the CPU budget is spent.
    Also the GPU's parity on every row the oracle computed."""
    import numpy as np
    import oracle
    import workloads as W
    w = head["w"]
    q, k, v = w.values("q"), w.values("k"), w.values("v")
    o_gpu, l_gpu = head["out"]
    chunks = [w.sample_rows]
    t_cpu, flops, done = 0.0, 0.0, 0
    worst = {"O": {"max_abs": 0.0, "rel_l2": 0.0}, "LSE": {"max_abs": 0.0, "rel_l2": 0.0}}
    first = None
    extra = W.more_query_rows(w.cfg, w.B, w.Hq, w.Nq, 64 * 512)
    ci = 0
    while True:
        rows = chunks[0] if ci == 0 else extra[(ci - 1) * 512:ci * 512]
        if len(rows) == 0:
            break
        t0 = time.perf_counter()
        O, L = oracle.ref_fwd_rows(q, k, v, rows, causal=True, scale=w.scale)
        dt = time.perf_counter() - t0
        t_cpu += dt
        flops += sum(4.0 * w.d * (int(i) + 1) for _, _, i in rows)
        done += len(rows)
        p = parity([("O", gather_rows(o_gpu, rows), O), ("LSE", gather_rows(l_gpu, rows), L)], "")
        for n in ("O", "LSE"):
            for mkey in ("max_abs", "rel_l2"):
                worst[n][mkey] = max(worst[n][mkey], p[n][mkey])
        if ci == 0:
            first = {"seconds": dt, "O": p["O"], "LSE": p["LSE"]}
        ci += 1
        if t_cpu >= args.cpu_seconds:
            break
    rate = flops / t_cpu
    full_s = head["flops"] / rate
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cores_available": _HOST_CORES,
            "sample": f"{done} query rows of the headline workload (the 512 seeded parity rows, then further "
                      f"seeded rows in chunks of 512 until {args.cpu_seconds:.0f} s of CPU), each against its "
                      f"own causal keys; fp64 numpy materialising the scores and weights; rate = causal "
                      f"algorithmic FLOPs of those rows / oracle seconds",
            "seconds": t_cpu, "rows": done,
            "parity_rows_512": first,
            "extrapolated_full_problem_seconds": full_s,
            "extrapolated_note": "extrapolated: full-problem FLOPs / the sample's rate (not run)",
            "gpu_vs_oracle_on_sample": worst,
            "gpu_speedup_vs_oracle": (head["flops"] / head["avg_s"]) / rate}


def row_fwd_small(args, fa):
    """Single-head non-causal fp32 forward (vector ALUs, float32 throughout)."""
    import oracle
    w, t, o, lse = fwd_workload(1)
    run = fa.prepare_fwd(t["q"], t["k"], t["v"], o, lse, causal=False, scale=w.scale)
    avg, tm = measure(run, max(20, args.steps), 5)
    flops = 4.0 * w.B * w.Hq * w.d * w.Nq * w.Nk
    out = {"workload": w.name, "tflops": flops / avg / 1e12, "timing": tm,
           "roofline": roofline("alu", flops, avg, "fa::fwd_f32_kernel<64>", flops_per_launch=flops,
                                note="launch-latency bound at this size: 4 workgroups")}
    if not args.no_parity:
        O, L = oracle.ref_fwd(w.values("q"), w.values("k"), w.values("v"), causal=False, scale=w.scale)
        out["parity"] = parity([("O", host(o), O), ("LSE", host(lse), L)], "full")
    return out


def row_fwd_causal_d64(args, fa):
    """Causal forward B4 H16 N2048 d64 bf16."""
    import oracle
    w, t, o, lse = fwd_workload(2)
    run = fa.prepare_fwd(t["q"], t["k"], t["v"], o, lse, causal=True, scale=w.scale)
    avg, tm = measure(run, args.steps, args.warmup)
    flops = 4.0 * w.B * w.Hq * w.d * causal_pairs(w.Nq, w.Nk)
    algo_bytes = 2 * (w.B * w.Hq * w.Nq * w.d * 2) + 2 * (w.B * w.Hkv * w.Nk * w.d * 2) + w.B * w.Hq * w.Nq * 4
    out = {"workload": w.name, "tflops": flops / avg / 1e12, "frac_of_peak": flops / avg / PEAK_BF16,
           "timing": tm,
           "roofline": roofline("mfma", flops, avg, "fa::fwd_ring_kernel<64, 4, 2, 1, true>",
                                "fwd_bf16_causal_d64_B4H16N2048", FWD_SOURCES, flops_per_launch=flops,
                                algorithmic_bytes_per_launch=algo_bytes)}
    if not args.no_parity:
        sl = (slice(0, 1), slice(0, 2))    # batch 0, heads 0-1 against the full oracle
        q, k, v = (w.values(n)[sl] for n in ("q", "k", "v"))
        O, L = oracle.ref_fwd(q, k, v, causal=True, scale=w.scale)
        out["parity"] = parity([("O", host(o[sl]), O), ("LSE", host(lse[sl]), L)], "batch 0, heads 0-1 (full rows)")
    return out


def row_fwd_fp8(args, fa):
    """The LLaMA-shaped causal forward with E4M3 inputs (per-tensor descales)."""
    import numpy as np
    import torch
    import oracle
    import workloads as W
    w = W.make_config(3)
    f8 = W.to_fp8(w)
    dev = {n: torch.from_numpy(c).to("cuda:0") for n, (c, _) in f8.items()}
    o = torch.empty((w.B, w.Hq, w.Nq, w.d), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda:0")
    run = fa.prepare_fwd_fp8(dev["q"], dev["k"], dev["v"], o, lse, f8["q"][1], f8["k"][1], f8["v"][1], causal=True,
                             scale=w.scale)
    avg, tm = measure(run, max(5, args.steps // 5), max(2, args.warmup // 2))
    flops = 4.0 * w.B * w.Hq * w.d * causal_pairs(w.Nq, w.Nk)
    out = {"workload": "llama_causal_fwd_B2_H32_N8192_d128_fp8_e4m3_kout", "tflops": flops / avg / 1e12,
           "frac_of_fp8_peak": flops / avg / PEAK_FP8, "timing": tm,
           "roofline": roofline("mfma", flops, avg, FP8_KERNEL, "fwd_fp8_causal_d128_B2H32N8192", FP8_SOURCES,
                                peak=PEAK_FP8,
                                flops_per_launch=flops, dtype="fp8 e4m3")}
    if not args.no_parity:
        vals = {n: oracle.e4m3_value(c) * s for n, (c, s) in f8.items()}
        rows = w.sample_rows
        O, L = oracle.ref_fwd_rows(vals["q"], vals["k"], vals["v"], rows, causal=True, scale=w.scale)
        out["parity"] = parity([("O", gather_rows(o, rows), O), ("LSE", gather_rows(lse, rows), L)],
                               "512 sampled rows; O carries the E4M3 rounding of the weights")
    return out


def row_fwd_bwd(args, fa, **override):
    import torch
    import oracle
    import workloads as W
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
    af, tf = measure(fa.prepare_fwd(q, k, v, o, lse, causal=True, scale=w.scale), n, 3)
    ab, tb = measure(fa.prepare_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal=True, scale=w.scale), n, 3)
    pairs = causal_pairs(w.Nq, w.Nk)
    ff = 4.0 * w.B * w.Hq * w.d * pairs
    fb = 10.0 * w.B * w.Hq * w.d * pairs
    name = w.name if not override else f"causal_fwd_bwd_B{w.B}_Hq{w.Hq}_Hkv{w.Hkv}_N{w.Nq}_d{w.d}_bf16"
    out = {"workload": name, "fwd_tflops": ff / af / 1e12, "fwd_frac_of_peak": ff / af / PEAK_BF16,
           "bwd_tflops": fb / ab / 1e12, "bwd_frac_of_peak": fb / ab / PEAK_BF16,
           "bwd_flop_convention": "10*B*H*d*pairs (five products, recompute included)",
           "fwd_bwd_tflops": (ff + fb) / (af + ab) / 1e12, "fwd_timing": tf, "bwd_timing": tb,
           "fwd_roofline": roofline("mfma", ff, af, "fa::fwd_ring_kernel<128, 8, 2, 1, true>", flops_per_launch=ff),
           "bwd_roofline": roofline("mfma", fb, ab, " + ".join(BWD_KERNELS) + " (one fa_bwd call)",
                                    "bwd_bf16_causal_d128_B2H16N4096" if not override
                                    else f"bwd_bf16_causal_gqa_d{w.d}_B{w.B}Hq{w.Hq}Hkv{w.Hkv}N{w.Nq}", BWD_SOURCES,
                                    flops_per_launch=fb)}
    if not args.no_parity:
        # one whole group of query heads (batch 0, K/V head 0) against the fp64 oracle
        g = w.Hq // w.Hkv
        sq, sk = (slice(0, 1), slice(0, g)), (slice(0, 1), slice(0, 1))
        qv, dov = w.values("q")[sq], w.values("do")[sq]
        kv, vv = w.values("k")[sk], w.values("v")[sk]
        O, L = oracle.ref_fwd(qv, kv, vv, causal=True, scale=w.scale)
        dQ, dK, dV = oracle.ref_bwd(qv, kv, vv, dov, causal=True, scale=w.scale)
        out["parity"] = parity([("O", host(o[sq]), O), ("LSE", host(lse[sq]), L), ("dQ", host(dq[sq]), dQ),
                                ("dK", host(dk[sk]), dK), ("dV", host(dv[sk]), dV)],
                               f"batch 0, query heads 0-{g - 1} with K/V head 0 (full rows)")
    return out


def decode_inputs():
    import torch
    import workloads as W
    w = W.make_config(4)
    t = upload(w)
    sl = torch.from_numpy(w.seqlens).to("cuda:0")
    return w, t, sl


def flush_buffer():
    """1 GiB (> the 256 MB Infinity Cache + L2s), read between launches to
    empty the caches of the previous launch's lines."""
    import torch
    flush = torch.zeros(1 << 28, dtype=torch.float32, device="cuda:0")
    flush.sum()
    torch.cuda.synchronize()
    return flush


_DECODE_REF = {}


def decode_reference(w):
    import oracle
    if "O" not in _DECODE_REF:
        _DECODE_REF["O"], _DECODE_REF["L"] = oracle.ref_decode(w.values("q"), w.values("k"), w.values("v"),
                                                               w.seqlens, scale=w.scale)
    return _DECODE_REF["O"], _DECODE_REF["L"]


def row_decode(args, fa):
    import numpy as np
    import torch
    w, t, sl = decode_inputs()
    q, k, v = t["q"], t["k"], t["v"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda:0")
    ws = fa.decode_workspace(q, k)
    run = fa.prepare_decode(q, k, v, sl, o, lse, ws, scale=w.scale)
    valid = int(w.seqlens.astype(np.int64).sum())
    nbytes = valid * w.Hkv * w.d * 2 * 2 + q.numel() * 2 + o.numel() * 2 + lse.numel() * 4
    n = max(10, args.steps // 2)
    aw = time_steps(run, n, 5)
    flush = flush_buffer()
    # caches emptied by reading the flush buffer: they then hold only clean lines
    sc = stats(time_launches(run, n, 2, before=lambda: flush.sum()))
    # caches filled with dirty lines first: the launch also pays for evicting them
    sd = stats(time_launches(run, n, 2, before=lambda: flush.fill_(1.0)))
    gbps = lambda st: nbytes / (st["median_us"] * 1e-6) / 1e9
    warm = nbytes / aw / 1e9
    out = {"workload": w.name, "valid_keys": valid, "algorithmic_bytes": nbytes,
           "cold_gbps": gbps(sc), "cold_frac_of_hbm": gbps(sc) * 1e9 / PEAK_HBM,
           "warm_gbps": warm, "warm_frac_of_hbm": warm * 1e9 / PEAK_HBM,
           "cold_after_writes_gbps": gbps(sd),
           "timing_cold": sc, "warm_per_step_us": aw * 1e6, "timing_cold_after_writes": sd,
           "roofline": roofline("hbm", nbytes, sc["median_us"] * 1e-6,
                                " + ".join(DEC_KERNELS),
                                "decode_gqa_B16Hq32Hkv8_N32768_d128", DEC_SOURCES, algorithmic_bytes_per_launch=nbytes,
                                timing="median of cache-cold launches"),
           "note": "graded: cold = caches emptied (by reading a 1 GiB buffer) before each launch; "
                   "warm = back-to-back launches; cold_after_writes = caches filled with dirty lines first"}
    if not args.no_parity:
        O, L = decode_reference(w)
        out["parity"] = parity([("O", host(o), O), ("LSE", host(lse), L)], "full (all 512 query rows)")
    return out


def row_decode_chunk(args, fa):
    """Chunk decode on the decode workload's cache: 8 new tokens per head
    (causal to each sequence's length), as when a large model checks 8 drafted
    tokens; bytes as decode (valid K/V once) plus the larger q, o and lse."""
    import numpy as np
    import torch
    import oracle
    import workloads as W
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
    flush = flush_buffer()
    sc = stats(time_launches(run, n, 2, before=lambda: flush.sum()))
    gbps = nbytes / (sc["median_us"] * 1e-6) / 1e9
    out = {"workload": "gqa_decode_chunk_B16_Hq32_Hkv8_Nq8_N32768_d128_bf16_causal", "valid_keys": valid,
           "algorithmic_bytes": nbytes, "cold_gbps": gbps, "cold_frac_of_hbm": gbps * 1e9 / PEAK_HBM,
           "tflops": flops / (sc["median_us"] * 1e-6) / 1e12, "timing_cold": sc,
           "roofline": roofline("hbm", nbytes, sc["median_us"] * 1e-6,
                                " + ".join(CHUNK_KERNELS), "decode_chunk_gqa_B16Hq32Hkv8_Nq8_N32768_d128",
                                DEC_SOURCES, algorithmic_bytes_per_launch=nbytes,
                                timing="median of cache-cold launches"),
           "note": "caches emptied (by reading a 1 GiB buffer) before each launch"}
    if not args.no_parity:
        O, L = oracle.ref_decode_chunk(w.values("q"), w.values("k"), w.values("v"), w.seqlens, causal=True,
                                       scale=w.scale)
        out["parity"] = parity([("O", host(o), O), ("LSE", host(lse), L)], "full (all 4096 query rows)")
    return out


def row_decode_paged(args, fa):
    """The decode workload with its cache in 64-key pages at seeded random
    positions of a page pool, reached through a block table."""
    import numpy as np
    import torch
    P = 64
    w, t, sl = decode_inputs()
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
    flush = flush_buffer()
    sc = stats(time_launches(run, n, 2, before=lambda: flush.sum()))
    gbps = nbytes / (sc["median_us"] * 1e-6) / 1e9
    out = {"workload": "gqa_decode_paged_B16_Hq32_Hkv8_N32768_d128_bf16_page64", "valid_keys": valid,
           "algorithmic_bytes": nbytes, "cold_gbps": gbps, "cold_frac_of_hbm": gbps * 1e9 / PEAK_HBM,
           "timing_cold": sc,
           "roofline": roofline("hbm", nbytes, sc["median_us"] * 1e-6,
                                " + ".join(DEC_KERNELS) + " (paged)", "decode_paged_gqa_B16Hq32Hkv8_N32768_d128_page64",
                                DEC_SOURCES, algorithmic_bytes_per_launch=nbytes,
                                timing="median of cache-cold launches"),
           "note": "64-key pages at seeded random pool positions; caches emptied (by reading a 1 GiB buffer) "
                   "before each launch"}
    if not args.no_parity:
        # the pages spell out the decode workload's cache: the decode oracle is the reference
        O, L = decode_reference(w)
        out["parity"] = parity([("O", host(o), O), ("LSE", host(lse)[:, :, 0], L)], "full (all 512 query rows)")
    return out


ROW_FUNCS = {
    "fwd_small": row_fwd_small, "fwd_causal_d64": row_fwd_causal_d64, "fwd_fp8": row_fwd_fp8,
    "fwd_bwd": row_fwd_bwd, "fwd_bwd_gqa": lambda a, f: row_fwd_bwd(a, f, Hq=32, Hkv=8),
    "decode": row_decode, "decode_chunk": row_decode_chunk, "decode_paged": row_decode_paged,
}


def headline_parity(head):
    """The GPU's headline output on the 512 sampled rows against the oracle."""
    import numpy as np
    import oracle
    w = head["w"]
    O, L = oracle.ref_fwd_rows(w.values("q"), w.values("k"), w.values("v"), w.sample_rows, causal=True,
                               scale=w.scale)
    o, lse = head["out"]
    return parity([("O", gather_rows(o, w.sample_rows), O), ("LSE", gather_rows(lse, w.sample_rows), L)],
                  "512 seeded sampled query rows")


def _pmc_per_launch(path, counter):
    """{kernel name: (counter value per launch, launches)} from a rocprofv3
    counter_collection.csv (rows of one dispatch are summed)."""
    import csv
    from collections import defaultdict
    per = defaultdict(lambda: defaultdict(float))
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                per[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return per


def pmc_summary(args):
    """HBM bytes per call of one target's kernels from a FETCH_SIZE and a
    WRITE_SIZE pass.  Each counter is scaled by what it reads for the three
    256 MiB calibration copies in the same run (FETCH_SIZE counts about half
    the bytes a copy reads on this part, WRITE_SIZE all it writes)."""
    import numpy as np
    tg = PMC_TARGETS[args.pmc_target]
    out = {"kernel": " + ".join(tg["kernels"]), "workload": tg["name"],
           "source_digest": source_digest(tg["sources"])}
    scale, per_call = {}, {}
    for counter, path in (("FETCH_SIZE", args.pmc_summary[0]), ("WRITE_SIZE", args.pmc_summary[1])):
        per = _pmc_per_launch(path, counter)
        copies = sorted((v for k, d in per.items() if "copyBuffer" in k for v in d.values()), reverse=True)[:3]
        if len(copies) < 3:
            raise SystemExit(f"{path}: the three calibration copies are missing (profile with --calibrate-copy)")
        scale[counter] = (256 << 10) / float(np.mean(copies))   # KiB a 256 MiB copy moves / KiB counted
        total, launches = 0.0, []
        for kname in tg["kernels"]:
            hits = [d for k, d in per.items() if k.startswith("void " + kname + "(") or k.startswith(kname + "(")]
            if len(hits) != 1:
                raise SystemExit(f"{path}: kernel {kname} found {len(hits)} times")
            vals = list(hits[0].values())
            total += float(np.mean(vals))
            launches.append(len(vals))
        per_call[counter] = total
        out[counter.lower() + "_kib_per_call"] = total
        out[counter.lower() + "_launches_counted"] = launches
    rd = per_call["FETCH_SIZE"] * 1024 * scale["FETCH_SIZE"]
    wr = per_call["WRITE_SIZE"] * 1024 * scale["WRITE_SIZE"]
    out["calibration"] = {"kernel": "__amd_rocclr_copyBuffer (torch copy_ of 256 MiB, 3 launches)",
                          "fetch_scale": scale["FETCH_SIZE"], "write_scale": scale["WRITE_SIZE"]}
    out.update(hbm_read_bytes_per_call=rd, hbm_write_bytes_per_call=wr, hbm_bytes_per_launch=rd + wr)
    if tg["read"] is not None:
        out.update(algorithmic_read_bytes=tg["read"], algorithmic_write_bytes=tg["write"],
                   read_over_algorithmic=rd / tg["read"], write_over_algorithmic=wr / tg["write"])
    out["note"] = tg["note"]
    base = ("cd /tmp && export TMPDIR=/tmp && timeout -k 10 300 rocprofv3 --pmc {c} -d $OUT/pmc_{c}_{t} "
            "-o run --output-format csv -- python3 $R/bench.py --only {o} --steps 5 --warmup 1 --no-parity --calibrate-copy"
            "   # R = repository root, OUT = any output directory")
    out["commands"] = [base.format(c=c, t=args.pmc_target, o=tg["only"]) for c in ("FETCH_SIZE", "WRITE_SIZE")] + [
        f"python3 bench.py --pmc-summary <FETCH_SIZE counter_collection.csv> <WRITE_SIZE counter_collection.csv> "
        f"--pmc-target {args.pmc_target}"]
    path = args.pmc_out or os.path.join(PROFILES, f"{tg['name']}_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def calibrate_copy():
    """Three plain 256 MiB device-to-device copies: known bytes for scaling
    the HBM traffic counters of the same profiled run."""
    import torch
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def main():
    global SETTLE_S
    args = parse_args()
    if args.pmc_summary:
        pmc_summary(args)
        return
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
    fa.load_library()   # raises if libfa.so is not built: there is no other path
    if args.calibrate_copy:
        calibrate_copy()

    if args.only in ROW_FUNCS:
        print(json.dumps({args.only: ROW_FUNCS[args.only](args, fa)}), flush=True)
        return
    if args.only == "ceilings":
        print(json.dumps({"measured_ceilings": ceilings()}), flush=True)
        return

    log("headline: causal forward B2 H32 N8192 d128 bf16 (1% key rows x8)")
    head = headline(args, fa)
    if args.only == "headline":
        print(json.dumps({"headline_tflops": head["flops"] / head["avg_s"] / 1e12, "timing": head["timing"]}),
              flush=True)
        return
    rows, ceil, cpu, hpar = {}, None, None, None
    if not args.headline_only:
        if not args.no_parity:
            hpar = headline_parity(head)
        for name in ROWS:
            log(f"row: {name}")
            rows[name] = ROW_FUNCS[name](args, fa)
            torch.cuda.empty_cache()
        if not args.no_ceilings:
            log("measured ceilings")
            ceil = ceilings()
        if not args.no_cpu_baseline:
            log("cpu baseline: fp64 oracle on sampled rows of the headline workload")
            cpu = cpu_baseline(args, head)

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
        "data": "synthetic (seeded N(0,1), bf16 round-to-nearest-even; 1% of key rows x8)",
        "config": {"workload": w.name, "B": w.B, "H": w.Hq, "N": w.Nq, "d": w.d, "causal": True,
                   "flops_per_step": head["flops"], "flop_convention": "4*B*H*d*N(N+1)/2"},
        "frac_of_peak": head["flops"] / head["avg_s"] / PEAK_BF16,
        "timing": head["timing"],
        "clock_settle_s": SETTLE_S,
        "roofline": head["roofline"],
        "parity": hpar,
        "cpu_baseline": cpu,
        "measured_ceilings": ceil,
        "rows": rows,
        "context": {"pages_claims": "2-4x faster and 10-20x less memory than standard attention; "
                                    "FlashAttention-3 1.5-2 PFLOP/s on NVIDIA H100 (other hardware, not a target)"},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
