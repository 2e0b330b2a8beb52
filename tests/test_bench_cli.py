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
