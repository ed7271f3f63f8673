"""Host-side checks of bench.py that need no GPU: the one-GPU contract (any
--gpus other than 1 exits with status 2 and says why, before importing torch
or touching a device) and the shape of the committed HBM-traffic file it
reads."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2
        assert "one GPU only" in r.stderr
        assert r.stdout == ""


def test_traffic_file_shape():
    t = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert set(t["per_launch"]) == {"gemm_4096x4096_b1", "gemm_4096x4096_b8"}
    assert abs(t["fetch_scale"] - 2.0) < 1e-3 and t["write_scale"] == 1.0
    for v in t["per_launch"].values():
        # single-pass streaming: within 15 % of the algorithmic bytes
        assert 1.0 <= (v["fetch_bytes"] + v["write_bytes"]) / v["alg_bytes"] < 1.15
    assert len(t["kernel_hash"]) == 16
