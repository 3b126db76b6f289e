"""bench.py's accounting and argument contract, on the CPU.

The algorithmic bytes behind the roofline object are checked against the
E=256 H=6144 I=2048 T=256 layer worked out by hand: every expert is hit by
8 of the 2048 routed slots, so the streaming gate_up reads each expert's
gate and up codes (2 x 2048 x 6144 bytes) and FP32 block scales
(2 x 16 x 48 x 4 bytes) once, and per slot one activation row with its
scales (6144 + 48 x 4 bytes) and one h row with its scales (2048 + 16 x 4
bytes).
"""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_algorithmic_bytes_of_the_t256_layer():
    import bench
    wl = SimpleNamespace(E=256, H=6144, I=2048, T=256, k=8)
    counts = np.full(256, 8, dtype=np.int64)
    w = bench.algorithmic_work(wl, counts)
    per_expert = 2 * 2048 * 6144 + 2 * 16 * 48 * 4
    assert per_expert == 25_171_968 == w["per_expert_gate_up_bytes"]
    per_slot = (6144 + 48 * 4) + (2048 + 16 * 4)
    g = w["gate_up"]["stream"]
    assert g["experts"] == 256 and g["rows"] == 2048
    assert g["bytes"] == 256 * per_expert + 2048 * per_slot == 6_461_325_312
    assert g["flops"] == 2 * 2048 * (2 * 2048) * 6144  # gate and up: 2 FLOPs per MAC
    assert w["gate_up"]["narrow"]["experts"] == 0 and w["gate_up"]["wide"]["experts"] == 0
    # whole path: gate, up and down codes and scales, BF16 rows in and out,
    # ids and weights
    down = 6144 * 2048 + 48 * 16 * 4
    assert w["path_bytes"] == 256 * (per_expert + down) + 256 * 6144 * 2 * 2 + 256 * 8 * 8
    assert w["path_flops"] == 2048 * 3 * 2 * 2048 * 6144


def test_tile_groups_follow_the_row_counts():
    import bench
    wl = SimpleNamespace(E=4, H=256, I=192, T=100, k=2)
    counts = np.array([0, 16, 17, 167], dtype=np.int64)
    w = bench.algorithmic_work(wl, counts)
    g = w["gate_up"]
    assert (g["stream"]["experts"], g["narrow"]["experts"], g["wide"]["experts"]) == (1, 1, 1)
    assert (g["stream"]["rows"], g["narrow"]["rows"], g["wide"]["rows"]) == (16, 17, 167)
    assert w["experts_hit"] == 3 and w["slots"] == 200
    # I = 192 is padded to Ip = 256
    assert w["per_expert_gate_up_bytes"] == 2 * 256 * 256 + 2 * 2 * 2 * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "--gpus must be 1" in r.stdout + r.stderr
