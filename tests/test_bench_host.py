"""Host-side checks of bench.py: the one-GPU guard and the profile summaries
written from rocprofv3 CSV output (synthetic CSVs; no GPU, no profiler)."""
import csv
import os
import subprocess
import sys


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write(path, rows, fields):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summaries_scale_counters_and_pair_the_column_reduce(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "fwd.md"))
    monkeypatch.setattr(bench, "BWD_TRAFFIC_FILE", str(tmp_path / "bwd.md"))
    M, N = 16384, 7168
    copy_kib = (8 * M * N + 2 * N) // 2 / 1024.0
    head = f"void addrms::{bench.HEADLINE_KERNEL}(addrms::FwdArgs)"
    bwd = f"void addrms::{bench.BWD_KERNEL}(addrms::BwdArgs)"
    red = "void addrms::dw_colreduce_vec_kernel<0>(float const*, float const*, int, int, float*, float*)"
    alg_r, alg_w = 4 * M * N + 2 * N, 4 * M * N
    bm, bn = 32768, 4096
    P = 768

    def counters(kind):
        # FETCH_SIZE reads half of a copy's bytes on this chip, WRITE_SIZE all
        half = kind == "FETCH_SIZE"
        rows = [("__amd_rocclr_copyBuffer", copy_kib / (2 if half else 1)),
                (head, (alg_r if half else alg_w) / 1024 / (2 if half else 1))]
        for _ in range(2):
            rows.append((bwd, ((2 * 2 * bm * bn) if half else (2 * bm * bn + P * bn * 4)) / 1024 /
                         (2 if half else 1)))
            rows.append(("void addrms::other_kernel()", 1.0))  # between the pair: skipped
            rows.append((red, ((P * bn * 4) if half else 4 * bn) / 1024 / (2 if half else 1)))
        return [{"Dispatch_Id": i + 1, "Kernel_Name": k, "Counter_Name": kind, "Counter_Value": v}
                for i, (k, v) in enumerate(rows)]

    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _write(str(tmp_path / "f" / "x_counter_collection.csv"), counters("FETCH_SIZE"), fields)
    _write(str(tmp_path / "w" / "x_counter_collection.csv"), counters("WRITE_SIZE"), fields)
    stats = [{"Name": head, "Calls": 2, "TotalDurationNs": 300000, "AverageNs": 150000.0,
              "MinNs": 149000, "MaxNs": 151000, "Percentage": 50.0},
             {"Name": bwd, "Calls": 2, "TotalDurationNs": 274000, "AverageNs": 137000.0,
              "MinNs": 136000, "MaxNs": 138000, "Percentage": 45.0}]
    _write(str(tmp_path / "t" / "x_kernel_stats.csv"), stats, list(stats[0].keys()))
    # per-dispatch trace: the headline's two dispatches (149 and 151 us), then
    # a later use of the same kernel (a per-call or in-place figure) that the
    # headline's average must leave out
    trace = [{"Dispatch_Id": k + 1, "Kernel_Name": head, "Start_Timestamp": 1000 * k * 1000,
              "End_Timestamp": 1000 * k * 1000 + d}
             for k, d in enumerate((149000, 151000, 400000))]
    _write(str(tmp_path / "t" / "x_kernel_trace.csv"), trace, list(trace[0].keys()))
    cmds = {"trace": "T", "fetch": "F", "write": "W", "headline_dispatches": 2}
    bench.summarize_profiles(str(tmp_path / "t"), str(tmp_path / "f"), str(tmp_path / "w"), cmds)

    fwd = (tmp_path / "fwd.md").read_text()
    assert "FETCH_SIZE is scaled by 2.0000 and WRITE_SIZE by 1.0000" in fwd
    assert f"- traffic_bytes_per_launch: {alg_r + alg_w}" in fwd
    assert "- kernel_avg_us_rocprof: 150.000" in fwd
    b = (tmp_path / "bwd.md").read_text()
    assert f"| column reduce (partial rows in; dw out) | {P * bn * 4} | {4 * bn} |" in b
    assert f"(here about {P} rows)" in b
    assert "main kernel average: 137.00 us" in b


def test_oracle_baselines_of_the_other_workloads():
    out = bench.cpu_baseline_configs(target_s=0.05)
    assert set(out) == {"rmsnorm_fwd_f32_256x4096", "add_rmsnorm_fwd_bf16_4096x4096",
                        "add_rmsnorm_fwd_bf16_decode_n8192_m512", "rmsnorm_bwd_bf16_32768x4096"}
    for name, r in out.items():
        assert 1 <= r["rows"] <= r["of_rows"] and r["rows_per_s"] > 0 and r["GBps"] > 0, name
        assert r["cores"] == 1


def test_row_sweep_summary_recovers_the_line(tmp_path):
    """Synthetic trace: every dispatch of shape (M, N) lasts t0 + bytes / B,
    the forward's and the probe's on lines of their own (warm-up calls 3 us
    slower, with copies interleaved); the summary must drop the warm-up calls
    and recover both lines."""
    t0, B = 1.7, 6200.0  # us, GB/s
    pt0, pB = 1.5, 6300.0  # the probe's line
    rows, did, ts = [], 0, 10_000_000
    name = ("void addrms::fwd_vec_kernel<addrms::bf16_t, addrms::bf16_t, 0, true, 0, 16, 1>"
            "(addrms::FwdArgs)")
    pname = ("void (anonymous namespace)::" + bench.ROW_SWEEP_PROBE_KERNEL
             + " -1, -1>((anonymous namespace)::PArgs, unsigned int*)")
    for N in bench.ROW_SWEEP_N:
        for M in bench.ROW_SWEEP_M:
            nb = 8 * M * N + 2 * N
            for kname, line in ((name, (t0, B, nb)), (pname, (pt0, pB, 8 * M * N))):
                for k in range(bench.ROW_SWEEP_WARMUP + bench.ROW_SWEEP_CALLS):
                    us = line[0] + line[2] / line[1] / 1e3 + (3.0 if k < bench.ROW_SWEEP_WARMUP else 0.0)
                    for kn, dur in (("__amd_rocclr_copyBuffer", 1.0), (kname, us)):
                        did += 1
                        rows.append({"Dispatch_Id": did, "Kernel_Name": kn, "Start_Timestamp": ts,
                                     "End_Timestamp": ts + int(round(dur * 1e3)),
                                     "Workgroup_Size_X": 1024, "Grid_Size_X": 1024 * M})
                        ts += 1_000_000
    _write(str(tmp_path / "t" / "rows_kernel_trace.csv"), rows, list(rows[0].keys()))
    out = str(tmp_path / "rows.md")
    bench.summarize_row_sweep(str(tmp_path / "t"), out, {"trace": "rocprofv3 ... --row-sweep"})
    text = open(out).read()
    assert text.count(f"Fit: t0 = {t0:.2f} us, B = {B:.0f} GB/s") == len(bench.ROW_SWEEP_N)
    assert text.count(f"Probe fit: t0 = {pt0:.2f} us, B = {pB:.0f} GB/s") == len(bench.ROW_SWEEP_N)
    assert "| 16384 | WPR 16, VPL 1 | 16384 x 1024 |" in text
