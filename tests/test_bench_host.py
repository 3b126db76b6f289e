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


def test_streamed_result_json():
    import json

    import bench
    import gen
    r = bench.streamed_result(gen.GLM_T4096, 6, 9_666_035_712, 1.2)
    json.dumps(r)
    assert r["steps"] == 6 and r["value"] == 4096 / 1.2 and r["dtype"].startswith("fp8_e4m3")
    assert abs(r["h2d_GBs"] - 6 * 9.666035712 / 1.2) < 1e-9


def test_two_call_step_work_is_the_sum_of_its_calls():
    import bench
    import gen
    wl = gen.GLM_T256
    rng = np.random.default_rng(0)
    ids = rng.integers(0, wl.E, (wl.T, wl.k)).astype(np.int32)
    one = bench.algorithmic_work(wl, bench.plan_counts(ids, wl.E))
    half = SimpleNamespace(**{**wl.__dict__, "T": 128})
    a = bench.algorithmic_work(half, bench.plan_counts(ids[:128], wl.E))
    b = bench.algorithmic_work(half, bench.plan_counts(ids[128:], wl.E))
    two = bench.add_work(a, b)
    assert two["path_flops"] == one["path_flops"] and two["slots"] == one["slots"] == wl.T * wl.k
    # two calls read the weights of the experts each hits
    assert two["path_bytes"] >= one["path_bytes"]
    g = bench.launch_work(two, "gate_up_stream", calls=2)
    assert g["rows"] == (a["gate_up"]["stream"]["rows"] + b["gate_up"]["stream"]["rows"]) / 2
    d = bench.launch_work(one, "down_wide")
    assert d["flops"] == 2 * one["down"]["wide"]["rows"] * 2048 * 6144


def test_profile_summaries_round_trip(tmp_path, monkeypatch):
    """summarize_profiles turns rocprofv3-shaped CSVs into the committed
    summaries, and read_traffic finds the scaled bytes of a kernel there."""
    import bench
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    tag = "glm_e256_t256"
    out = tmp_path / "prof"

    def write_pmc(sub, counter, rows):
        d = out / sub / "host"
        d.mkdir(parents=True)
        with open(d / "pmc_counter_collection.csv", "w") as f:
            f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
            for i, (kern, val) in enumerate(rows):
                f.write(f'{i},"{kern}",{counter},{val}\n')

    write_pmc("copy_fetch", "FETCH_SIZE", [("void at::native::copyBuffer(char*)", 524288.0)])
    write_pmc("copy_write", "WRITE_SIZE", [("void at::native::copyBuffer(char*)", 1048576.0)])
    k = "void moe::gate_up_stream_kernel<5>(moe::GateUpArgs)"
    write_pmc(f"fetch_{tag}", "FETCH_SIZE", [(k, 1000.0), (k, 1002.0)])
    write_pmc(f"write_{tag}", "WRITE_SIZE", [(k, 10.0), (k, 10.0)])
    d = out / f"kt_{tag}" / "host"
    d.mkdir(parents=True)
    with open(d / "kt_kernel_stats.csv", "w") as f:
        f.write("Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs\n")
        f.write(f'"{k}",10,9500000,950000,60.0,940000,960000\n')
    with open(d / "kt_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for i, dur in enumerate((990000, 940000, 945000)):
            f.write(f'"{k}",{i * 10**7},{i * 10**7 + dur}\n')
    assert bench.summarize_profiles(str(out)) == 0
    stats = (tmp_path / "profiles" / f"kernel_stats_{tag}.md").read_text()
    assert "| 950.0 | 945.0 | 940.0 | 960.0 |" in stats  # average, trace median, min, max
    # FETCH scaled by 2 (the copy reads half its bytes), WRITE by 1
    assert bench.read_traffic("gate_up_stream_kernel", tag) == (1001.0 * 2 + 10.0) * 1024
    assert (tmp_path / "profiles" / f"kernel_stats_{tag}.md").exists()


def test_pipe_summary(tmp_path, monkeypatch):
    """The memory-pipe summary turns the three counter passes into per-kernel
    fractions (MFMA busy over C x 1024 SIMDs, waiting over wave time)."""
    import bench
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    (tmp_path / "profiles").mkdir()
    tag = "probe_e8_t4096"
    k = "void moe::gate_up_wide_kernel<false>(moe::GateUpArgs)"
    gui = 8 * 1000.0  # one XCD active for 1000 cycles
    values = {
        "pipe_a": {"SQ_WAVE_CYCLES": 2000.0, "SQ_WAIT_ANY": 500.0, "SQ_WAIT_INST_ANY": 800.0,
                   "SQ_WAIT_INST_LDS": 100.0, "SQ_ACTIVE_INST_LDS": 150.0, "SQ_ACTIVE_INST_VALU": 900.0,
                   "SQ_ACTIVE_INST_VMEM": 80.0, "GRBM_GUI_ACTIVE": gui},
        "pipe_b": {"SQ_LDS_BANK_CONFLICT": 10.0, "SQ_LDS_IDX_ACTIVE": 76800.0,
                   "SQ_VALU_MFMA_BUSY_CYCLES": 512000.0, "TA_TA_BUSY": 128000.0,
                   "TA_ADDR_STALLED_BY_TC_CYCLES": 0.0, "TD_TD_BUSY": 192000.0, "TD_TC_STALL": 25600.0,
                   "GRBM_GUI_ACTIVE": gui},
        "pipe_c": {"TCP_TCC_READ_REQ_LATENCY": 30000.0, "TCP_TCC_READ_REQ": 100.0,
                   "TCP_PENDING_STALL_CYCLES": 0.0, "SQ_INSTS_LDS": 100.0, "SQ_INSTS_VALU": 600.0,
                   "SQ_INSTS_MFMA": 100.0, "SQ_INSTS_VMEM_RD": 50.0, "GRBM_GUI_ACTIVE": gui},
    }
    out = tmp_path / "prof"
    for p, cs in values.items():
        d = out / f"{p}_{tag}" / "host"
        d.mkdir(parents=True)
        with open(d / "pmc_counter_collection.csv", "w") as f:
            f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
            for c, v in cs.items():
                f.write(f'0,"{k}",{c},{v}\n')
    cmds = bench.profile_commands(tag)
    assert bench._pipe_summary(str(out), tag, cmds, "x") == 1
    text = (tmp_path / "profiles" / f"pipe_{tag}.md").read_text()
    # MFMA busy 0.5, waiting 0.4, valu 0.45, lds 0.075, vmem 0.04, LDS busy 0.3, conflicts 0.1,
    # TA 0.5, TD 0.75, TD stalled 0.1, latency 300 cycles, 5 VALU per MFMA
    assert ("| `gate_up_wide_kernel` | 0.500 | 0.400 | 0.450 | 0.075 | 0.040 | 0.300 | 0.100 | 0.500 | "
            "0.750 | 0.100 | 300 | 5.0 |") in text


def test_path_object_peaks():
    """The path fraction takes the FP8 peak for W8A8 and the BF16 peak for
    the W8A16 decode path."""
    import bench
    work = {"path_bytes": 8e9, "path_flops": 2.5e12, "experts_hit": 1}
    w8 = bench.path_object(work, 1.0, None)
    w16 = bench.path_object(work, 1.0, None, a16=True)
    assert abs(w8["hbm_frac"] - 1.0) < 1e-12
    assert abs(w8["mfma_frac"] - 0.5) < 1e-12 and abs(w16["mfma_frac"] - 1.0) < 1e-12
    assert w16["mfma_peak_TFLOPs"] == bench.PEAK_BF16_TFLOPS
