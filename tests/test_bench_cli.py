"""The benchmark's host-side contract, without a GPU: one GPU's share only (a request for more GPUs
exits with a message and status 2), and the committed HBM-traffic summaries carry what the roofline
record needs (per-dispatch counters, the copy calibration, the commands that produced them)."""
import glob
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_summaries_are_complete():
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_traffic.json")))
    assert paths, "no traffic summaries committed"
    for p in paths:
        d = json.load(open(p))
        for key in ("kernel", "workload", "commands", "fetch_kib_per_dispatch", "write_kib_per_dispatch",
                    "fetch_scale", "write_scale", "bytes_per_launch", "csrc_sha256_16"):
            assert key in d, f"{os.path.basename(p)}: no {key}"
        assert any("--pmc FETCH_SIZE" in c for c in d["commands"]) and any("--pmc WRITE_SIZE" in c for c in d["commands"])
        # bytes = counters x calibration of a plain copy of known size
        want = d["fetch_kib_per_dispatch"] * d["fetch_scale"] + d["write_kib_per_dispatch"] * d["write_scale"]
        assert abs(d["bytes_per_launch"] - want) <= 1e-6 * want


def test_trace_summary_reports_the_timed_window(tmp_path):
    """--summarize-trace: every dispatch in the statistics table, and the average over the last K dispatches of
    the dominant kernel (the timed steps) beside it, from rocprofv3's kernel-trace CSV columns."""
    sys.path.insert(0, ROOT)
    import bench
    d = tmp_path / "kt"
    d.mkdir()
    (d / "run_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void mk::k_fused<X>(mk::FusedArgs)",5,5000,1000,99.0,500,1500,0\n')
    durs = [1500, 1200, 900, 800, 600]   # the first call and a warm-up, then three timed steps
    rows = ['"Kernel_Name","Start_Timestamp","End_Timestamp"']
    t = 1000
    for du in durs:
        rows.append(f'"void mk::k_fused<X>(mk::FusedArgs)",{t},{t + du}')
        rows.append(f'"other_kernel",{t + du + 10},{t + du + 20}')
        t += 10000
    (d / "run_kernel_trace.csv").write_text("\n".join(rows) + "\n")
    out = tmp_path / "summary.md"
    bench.summarize_trace(str(d), "tiny", "fused", 3, path=str(out))
    text = out.read_text()
    assert "| `void mk::k_fused<X>(mk::FusedArgs)` | 5 |" in text
    assert "| 3 | 0.8 | " in text      # (900 + 800 + 600) / 3 ns = 0.77 us, printed to one decimal
    assert "rocprofv3 --kernel-trace --stats" in text
