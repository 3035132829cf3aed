"""Host logic of bench.py that needs no GPU: the rocprofv3 counter summary
(per-call HBM bytes of a target's kernels, scaled by the calibration copies)."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        d = 0
        for kernel, values in rows:
            for v in values:
                d += 1
                # a dispatch may be reported in several rows (one per instance); they add up
                w.writerow([d, kernel, counter, v / 4])
                w.writerow([d, kernel, counter, 3 * v / 4])


def test_pmc_summary_scales_by_the_copies_and_sums_the_call(tmp_path):
    dq = "void fa::bwd_dq_kernel<128, true, float>(unsigned short const*, float*)"
    dkdv = "void fa::bwd_dkdv_kernel<128, true, float>(unsigned short const*, float*)"
    # FETCH_SIZE reads half of what a 256 MiB copy moves, WRITE_SIZE all of it;
    # a small unrelated copy and an unrelated kernel must not count
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", [131072, 131072, 131072, 9.0]),
                                            (dq, [1000.0, 1400.0]), (dkdv, [3000.0]),
                                            ("void fa::fwd_ring_kernel<128, 8, 2, 1, true>(int)", [5.0])])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", [262144, 262144, 262144]),
                                            (dq, [500.0]), (dkdv, [600.0, 800.0])])
    out = tmp_path / "t.json"
    subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--pmc-summary", str(tmp_path / "f.csv"),
                    str(tmp_path / "w.csv"), "--pmc-target", "fwd_bwd", "--pmc-out", str(out)],
                   check=True, capture_output=True)
    t = json.loads(out.read_text())
    assert t["calibration"]["fetch_scale"] == 2.0 and t["calibration"]["write_scale"] == 1.0
    assert t["fetch_size_kib_per_call"] == 1200.0 + 3000.0
    assert t["write_size_kib_per_call"] == 500.0 + 700.0
    assert t["hbm_read_bytes_per_call"] == 4200.0 * 1024 * 2
    assert t["hbm_write_bytes_per_call"] == 1200.0 * 1024
    assert t["hbm_bytes_per_launch"] == t["hbm_read_bytes_per_call"] + t["hbm_write_bytes_per_call"]
    # config 5: B2 H16 N4096 d128; five bf16 inputs and fp32 lse read, three fp32 gradients written
    assert t["algorithmic_read_bytes"] == 5 * 2 * 16 * 4096 * 128 * 2 + 2 * 16 * 4096 * 4
    assert t["algorithmic_write_bytes"] == 3 * 2 * 16 * 4096 * 128 * 4
    assert len(t["source_digest"]) == 16


def test_pmc_summary_refuses_a_run_without_calibration(tmp_path):
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [("void fa::fwd_ring_kernel<128, 8, 2, 1, true>(int)", [5.0])])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [("void fa::fwd_ring_kernel<128, 8, 2, 1, true>(int)", [5.0])])
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--pmc-summary", str(tmp_path / "f.csv"),
                        str(tmp_path / "w.csv"), "--pmc-out", str(tmp_path / "t.json")], capture_output=True, text=True)
    assert r.returncode != 0 and "calibration copies" in (r.stderr + r.stdout)


def test_committed_traffic_files_describe_their_targets():
    """Every profiles/<workload>_traffic.json that bench.py reads names the
    kernels and workload of its --pmc-target, and carries the per-call bytes,
    the calibration scales and the commands that made it."""
    sys.path.insert(0, ROOT)
    import bench
    seen = 0
    for target, tg in bench.PMC_TARGETS.items():
        path = os.path.join(ROOT, "profiles", f"{tg['name']}_traffic.json")
        if not os.path.exists(path):
            continue
        seen += 1
        with open(path) as f:
            t = json.load(f)
        assert t["workload"] == tg["name"], target
        assert t["kernel"] == " + ".join(tg["kernels"]), target
        assert t["hbm_bytes_per_launch"] == t["hbm_read_bytes_per_call"] + t["hbm_write_bytes_per_call"], target
        assert t["hbm_read_bytes_per_call"] > 0 and t["hbm_write_bytes_per_call"] > 0, target
        assert 1.5 < t["calibration"]["fetch_scale"] < 2.5 and 0.8 < t["calibration"]["write_scale"] < 1.2, target
        assert any(f"--pmc-target {target}" in c for c in t["commands"]), target
        assert len(t["source_digest"]) == 16, target
    assert seen >= 4


def test_bench_refuses_more_than_one_gpu():
    """One GPU only: --gpus N with N > 1 exits with a message before touching a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""
