"""bench.py's contract on the host: the one-GPU refusal, the algorithmic bytes behind
roofline.achieved (hand-counted on a tiny layer), and the HBM-traffic figure, which is reported
only while the profiled kernel source is the one in the tree."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_algorithmic_bytes_hand_count():
    # d = 64, f = 32, E = 4, k = 2, T = 2 tokens; experts 0 and 2 touched (U = 2), 4 pairs
    counts = np.array([3, 0, 1, 0])
    b = bench.algorithmic_bytes(counts, T=2, d=64, f=32, k=2, E=4)
    assert b["U"] == 2
    # gate/up: 2 experts x (32 + 32) rows x 64 inputs x 2 B = 16384; x rows 4 x 64 x 2 = 512; h rows 4 x 32 x 2 = 256
    assert b["gateup"] == 16384 + 512 + 256
    # down: 2 x 64 x 32 x 2 = 8192; h rows 256; y_perm rows 4 x 64 x 4 B = 1024
    assert b["down"] == 8192 + 256 + 1024
    # layer: 2 experts x 3 matrices (24576) + router 4 x 64 x 2 (512) + x in and y out 2 x 2 x 64 x 2 (512)
    assert b["layer"] == 24576 + 512 + 512
    # a shared expert adds one touched expert and T rows; int4 weights are 0.5 B + a bf16 scale per 128
    s = bench.algorithmic_bytes(counts, T=2, d=64, f=32, k=2, E=4, w_bytes=0.5 + 2 / 128, shared=True)
    assert s["U"] == 3
    assert s["gateup"] == 3 * 2 * 32 * 64 * (0.5 + 2 / 128) + 6 * 64 * 2 + 6 * 32 * 2


def test_traffic_figure_follows_the_profiled_source(tmp_path):
    src = "expert_offload_cache_amd/csrc/ffn_gemv_ks.hip"
    with open(bench.TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    # the committed counters were taken on the kernel source as it stands
    assert bench.traffic_for(src) == rec["hbm_bytes_per_launch"]
    assert 2.0e8 < rec["hbm_bytes_per_launch"] < 4.0e8
    changed = tmp_path / "ffn_gemv_ks.hip"
    with open(os.path.join(ROOT, src), "rb") as fh:
        changed.write_bytes(fh.read() + b"\n// changed\n")
    assert bench.traffic_for(str(changed)) is None
