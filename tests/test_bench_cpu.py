"""Host logic of bench.py, on the CPU: the roofline definition (max of the
HBM and transcendental times over the kernel time), the issue rates it reads,
the rocprofv3 summaries (traffic scaled by a copy of known size, the kernel
trace grouped by launch shape, the LDS probe table) on synthetic counter
files, the LDS probe's offset patterns, and the one-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from selective_state_space_ss_amd.workloads import WORKLOADS  # noqa: E402


def test_scan_roofline_is_max_of_hbm_and_exp_time():
    w = WORKLOADS["mamba2p8b"]
    rates = (3.8e13, 1.9e13, "test")
    r = bench.scan_roofline(w, 331.0, rates)
    ct = 8 * 5120 * 2048
    assert r["algorithmic_bytes"] == 677748736
    assert r["transcendentals"] == ct * (16 + 2 + 2) == 1677721600
    t = 331e-6
    hbm, exp = 677748736 / 8e12, 1677721600 / 1.9e13
    assert r["hbm_frac"] == pytest.approx(hbm / t, abs=1e-4)
    assert r["exp_frac"] == pytest.approx(exp / t, abs=1e-4)
    assert r["frac"] == pytest.approx(max(hbm, exp) / t, abs=1e-4)
    fma = ct * (4 * 16 + 6 + 3)
    assert r["issue_frac"] == pytest.approx((exp + fma / 3.8e13) / t, abs=1e-4)
    # without the gate the exp count drops by two per channel-token
    w2 = WORKLOADS["packed_reset"]
    assert bench.scan_work(w2)["trans"] == 4 * 2048 * 8192 * (16 + 2)


def test_decode_roofline_is_hbm_fraction():
    w = WORKLOADS["decode"]
    r = bench.decode_roofline(w, 30.0)
    assert r["algorithmic_bytes"] == 178642944
    assert r["hbm_frac"] == pytest.approx(178642944 / 30e-6 / 8e12, abs=1e-4)


def test_issue_rates_come_from_the_committed_probe():
    fma, exp, src = bench.issue_rates()
    with open(os.path.join(ROOT, "profiles", "issue_rates_gfx950.json")) as f:
        j = json.load(f)
    assert (fma, exp) == (j["fma_lane_ops_per_s"], j["exp2_lane_ops_per_s"])
    assert src == os.path.join("profiles", "issue_rates_gfx950.json")


def _counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for d, k, c, v in rows:
            wr.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_summarize_traffic_scales_each_counter_by_the_copy(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    scan = "void ss::scan_fwd_kernel<bf16_t, 16>(ss::ScanParams)"
    dec = "void ss::state_update_kernel<bf16_t>(ss::UpdateParams)"
    copy = "__amd_rocclr_copyBuffer"
    # FETCH_SIZE reads half the copied bytes, WRITE_SIZE all of them
    _counter_csv(str(tmp_path / "f" / "p" / "f_counter_collection.csv"),
                 [(1, copy, "FETCH_SIZE", 3), (2, copy, "FETCH_SIZE", 131072), (3, scan, "FETCH_SIZE", 1000),
                  (4, dec, "FETCH_SIZE", 50), (5, scan, "FETCH_SIZE", 1002)])
    _counter_csv(str(tmp_path / "w" / "p" / "w_counter_collection.csv"),
                 [(2, copy, "WRITE_SIZE", 262144), (3, scan, "WRITE_SIZE", 500), (5, scan, "WRITE_SIZE", 700)])
    bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"))
    t = json.loads(out.read_text())
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["write_scale"] == pytest.approx(1.0)
    assert t["fetch_bytes_per_scan"] == pytest.approx(1001 * 1024 * 2.0)
    assert t["write_bytes_per_scan"] == pytest.approx(600 * 1024)
    assert t["traffic_bytes_per_scan"] == pytest.approx(1001 * 2048 + 600 * 1024)
    assert t["kernel_source_digest"] == bench.kernel_source_digest()


def test_summarize_trace_rows_per_launch_shape(tmp_path, capsys):
    path = tmp_path / "kt" / "kt_kernel_trace.csv"
    os.makedirs(path.parent)
    names = ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Workgroup_Size_X", "Workgroup_Size_Y",
             "Workgroup_Size_Z", "Start_Timestamp", "End_Timestamp"]
    k = "void ss::(anonymous namespace)::scan_fwd_kernel<ss::bf16_t, 16>(ss::ScanParams)"
    rows = [(k, 655360, 100, 400), (k, 655360, 1000, 1200), (k, 196608, 0, 60)]
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(names)
        for name, grid, s, e in rows:
            wr.writerow([name, grid, 1, 1, 512, 1, 1, s, e])
    bench.summarize_trace(str(tmp_path / "kt"))
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("| `")]
    assert len(lines) == 2
    big = next(ln for ln in lines if "| 655360 |" in ln)
    small = next(ln for ln in lines if "| 196608 |" in ln)
    assert "| 2 | 250 |" in big and "ss::scan_fwd_kernel<ss::bf16_t, 16>" in big
    assert "| 1 | 60 |" in small


def test_lds_patterns_are_in_bounds_and_aligned():
    pats = bench.lds_patterns()
    assert len({p[0] for p in pats}) == len(pats)
    for name, width, write, offs in pats:
        assert width in (4, 8, 16) and write in (0, 1)
        assert len(offs) == 64
        assert all(0 <= o <= 65536 - 16 and o % width == 0 for o in offs), name


def test_summarize_lds_table(tmp_path, capsys):
    pats = bench.lds_patterns()
    rows = [(1, "lds_probe_kernel<16, false>", "SQ_LDS_BANK_CONFLICT", 0)]  # the warm-up launch
    for i in range(len(pats)):
        rows.append((i + 2, "lds_probe_kernel<16, false>", "SQ_LDS_BANK_CONFLICT", 1000 * i))
        rows.append((i + 2, "lds_probe_kernel<16, false>", "SQ_INSTS_LDS", 1256))
    _counter_csv(str(tmp_path / "l" / "p" / "l_counter_collection.csv"), rows)
    bench.summarize_lds(str(tmp_path / "l"))
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("| ") and "---" not in ln][1:]
    assert len(lines) == len(pats)
    for i, ln in enumerate(lines):
        assert ln.startswith(f"| {pats[i][0]} |") and ln.endswith(f"| {float(i):.2f} |")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_percentiles_nearest_rank():
    each = [float(v) for v in range(1, 51)]          # 1 .. 50 us, shuffled order must not matter
    p = bench.percentiles(each[::-1])
    assert p == {"p10_us": 6.0, "median_us": 25.0, "p90_us": 45.0}
    assert bench.percentiles([7.0]) == {"p10_us": 7.0, "median_us": 7.0, "p90_us": 7.0}


def test_step_decode_launches_follow_the_scan(tmp_path, capsys):
    path = tmp_path / "kt" / "kt_kernel_trace.csv"
    os.makedirs(path.parent)
    names = ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Workgroup_Size_X", "Workgroup_Size_Y",
             "Workgroup_Size_Z", "Start_Timestamp", "End_Timestamp"]
    scan = "void ss::(anonymous namespace)::scan_fwd_kernel<ss::bf16_t, 16, 8, 16, true, false, 0, 0, 16>(ss::ScanParams)"
    dec = "void ss::(anonymous namespace)::state_update_kernel<ss::bf16_t, 1, true, true>(ss::UpdateParams)"
    rows = [(scan, 0, 300), (dec, 302, 330),          # a step: counted (28)
            (scan, 400, 700), (dec, 705, 735),        # a step: counted (30)
            (dec, 740, 770),                          # a warm launch after a decode: not counted
            (scan, 800, 1100), (dec, 900, 1000),      # overlapping the scan (two streams): not counted
            ]
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(names)
        for name, s, e in rows:
            wr.writerow([name, 1, 1, 1, 256, 1, 1, s, e])
    assert sorted(bench.step_launches([str(path)])) == [28, 30]
    bench.summarize_trace(str(tmp_path / "kt"))
    out = capsys.readouterr().out
    assert "In the bench step: 2 decode launches" in out and "mean 29 ns" in out


def test_summarize_counters_sums_instances_then_takes_the_median(tmp_path, capsys):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = []
    # three dispatches of the scan, two counter instances each; one copy dispatch that must be ignored
    for d, vals in ((1, (10.0, 1.0)), (2, (20.0, 2.0)), (3, (40.0, 4.0))):
        for v in vals:
            rows.append({"Dispatch_Id": d, "Kernel_Name": "void ss::scan_fwd_kernel<x>(p)",
                         "Counter_Name": "SQ_INSTS_VALU", "Counter_Value": v})
    rows.append({"Dispatch_Id": 4, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "SQ_INSTS_VALU",
                 "Counter_Value": 1e9})
    os.makedirs(tmp_path / "p1")
    with open(tmp_path / "p1" / "p1_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        w.writerows(rows)
    bench.summarize_counters([str(tmp_path / "p1")], "scan_fwd_kernel")
    out = capsys.readouterr().out
    # per dispatch 11, 22, 44 -> median 22
    assert "| SQ_INSTS_VALU | 22 | 3 |" in out
    assert "copyBuffer" not in out


def test_single_thread_oracle_timing_and_host_info():
    r = bench.cpu_single_thread(names=("tiny_fp32",), budget_s=0.1)["tiny_fp32"]
    w = WORKLOADS["tiny_fp32"]
    assert r["rows"] == w.channels and r["channel_tokens"] == w.channels * w.seqlen
    assert r["wall_s"] > 0 and r["channel_tokens_per_s"] > 0 and r["GB_s"] > 0
    h = bench.host_cpu()
    assert h["nproc"] >= 1 and h["affinity_cpus"] >= 1 and isinstance(h["cpu_model"], str)
