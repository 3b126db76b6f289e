#!/usr/bin/env python3
"""Benchmark: input tokens/s of the routed-expert FP8 MoE prefill layer on one
MI355X, with each workload's dominant kernel against its roofline and the CPU
oracle beside it.

A step is one pass of the whole path (plan, quantise, gate_up, down,
combine) over one batch of seeded synthetic input already resident in HBM.
Default: the GLM-class layer (E=256, top-8, H=6144, I=2048, 9.002 GiB of FP8
weights and FP32 block scales) with T=8192 rows in one call, Zipf(1.2)
expert popularity (8 experts never chosen), sigmoid top-8 routing, routed
scale 2.5 and 1% outlier rows x100: the largest configuration, where the
256-row tile GEMMs run on the matrix cores.  The same layer at T=8192 as two
4096-row calls, at T=4096 (uniform routing logits) and at T=256 (the
HBM-bound small batch) are reported as sub-objects of the same line, each
with its own dominant-launch roofline.

Per workload:
  - ms_per_step / tokens_per_s: W warmup steps, then K steps back to back,
    wall clock between two device synchronisations;
  - stages_ms: five untimed steps with HIP events at every launch boundary;
    they name the dominant launch, whose time the timed steps then record
    with two events per pass on the run stream (roofline object);
  - protocol: the measurement method of "ktransformers #2245" (Real-checkpoint
    measurements): per-call HIP events, median over `--protocol-calls` calls,
    each call's complete output compared bit for bit with the first one's;
    before every call a 512 MiB buffer is written (outside the events) so the
    256 MiB MALL holds none of the layer.

Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense BF16 MFMA, TFLOP/s (the W8A16 decode path)
METRIC = "input tokens/sec per MoE layer (1 MI355X) + % FP8 MFMA peak / % HBM peak"
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCE = os.path.join(ROOT, "fp8_blockwise_routed_amd", "csrc", "moe_kernels.hip")
MALL_FLUSH_BYTES = 512 << 20

HEADLINE = "glm_e256_k8_h6144_i2048_t8192_zipf"
# sub-objects of the default line: (key, workload, rows per call or None)
SUBS = (("t8192_zipf_2x4096", HEADLINE, 4096),
        ("t4096_uniform", "glm_e256_k8_h6144_i2048_t4096_uniform", None),
        ("t256", "glm_e256_k8_h6144_i2048_t256", None))

# library timing stage -> kernel launched in it
KERNELS = {
    "gate_up_stream": "gate_up_stream_kernel",
    "gate_up_narrow": "gate_up_narrow_kernel",
    "gate_up_wide": "gate_up_wide_kernel",
    "down_stream": "down_stream_kernel",
    "down_wide": "down_wide_kernel",
    "combine": "combine_kernel",
}
DESCRIBE = {
    "gate_up_stream": "gate_up_stream_kernel (experts with 1..16 rows)",
    "gate_up_narrow": "gate_up_narrow_kernel (experts with 17..128 rows)",
    "gate_up_wide": "gate_up_wide_kernel (experts with more than 128 rows)",
    "down_stream": "down_stream_kernel (experts with 1..16 rows)",
    "down_wide": "down_wide_kernel (experts with more than 16 rows: 128- and 256-row tiles)",
    "combine": "combine_kernel",
    "decode_gate_up": "gate_up_a16_kernel (W8A16 decode, every expert hit)",
}

# rocprofv3 runs whose CSV output --summarize-profiles reads (repository root)
# the bench's own warmup and timed steps, so the traced durations are those the
# timed steps see (the first few launches of a fresh process run slower)
_BENCH1 = "python3 bench.py --cpu-tokens 0 --protocol-calls 0 --no-peaks"
PROFILED = {  # tag -> workload
    "glm_e256_t8192_zipf": HEADLINE,
    "glm_e256_t4096_uniform": "glm_e256_k8_h6144_i2048_t4096_uniform",
    "glm_e256_t256": "glm_e256_k8_h6144_i2048_t256",
    "probe_e8_t4096": "probe_e8_k8_h6144_i2048_t4096",
    "slice_e160_t1024": "slice_e160_k8_h5120_i192_t1024",
    "glm_e256_t4096_router": "glm_e256_k8_h6144_i2048_t4096_uniform",
}
PROFILE_ARGS = {"glm_e256_t4096_router": " --router"}  # extra bench arguments of a tag
TITLES = {
    "glm_e256_t8192_zipf": "GLM-class layer E=256 top-8 H=6144 I=2048, T=8192 rows in one call, Zipf(1.2) routing",
    "glm_e256_t4096_uniform": "GLM-class layer E=256 top-8 H=6144 I=2048, T=4096 rows, uniform routing logits",
    "glm_e256_t256": "GLM-class layer E=256 top-8 H=6144 I=2048, T=256 rows",
    "probe_e8_t4096": "compute-bound probe: E=8, every token to all 8 experts, H=6144 I=2048, T=4096",
    "slice_e160_t1024": "tensor-sliced share E=160 top-8 H=5120 I=192 (padded to 256), T=1024",
    "glm_e256_t4096_router": "GLM-class layer E=256 top-8 H=6144 I=2048, T=4096 rows from router logits",
}
MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_BUSY_CYCLES GRBM_GUI_ACTIVE"
# where the tile kernels' cycles go: three passes within rocprofv3's per-block
# counter limits (8 SQ, 2 TA, 2 TD, 4 TCP, 2 GRBM)
PIPE_COUNTERS = {
    "pipe_a": "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS "
              "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_VMEM GRBM_GUI_ACTIVE",
    "pipe_b": "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES TA_TA_BUSY "
              "TA_ADDR_STALLED_BY_TC_CYCLES TD_TD_BUSY TD_TC_STALL GRBM_GUI_ACTIVE",
    "pipe_c": "TCP_TCC_READ_REQ_LATENCY TCP_TCC_READ_REQ TCP_PENDING_STALL_CYCLES SQ_INSTS_LDS SQ_INSTS_VALU "
              "SQ_INSTS_MFMA SQ_INSTS_VMEM_RD GRBM_GUI_ACTIVE",
}


# raw rocprofv3 output of the profile runs (read back by --summarize-profiles)
PROF_RAW = "rocprof_raw"


def profile_commands(tag):
    b = f"{_BENCH1} --workload {PROFILED[tag]}{PROFILE_ARGS.get(tag, '')}"
    return {
        "trace": f"rocprofv3 --kernel-trace --stats -f csv -d {PROF_RAW}/kt_{tag} -o kt -- {b}",
        "fetch": f"rocprofv3 --pmc FETCH_SIZE -f csv -d {PROF_RAW}/fetch_{tag} -o pmc -- {b}",
        "write": f"rocprofv3 --pmc WRITE_SIZE -f csv -d {PROF_RAW}/write_{tag} -o pmc -- {b}",
        "mfma": f"rocprofv3 --pmc {MFMA_COUNTERS} -f csv -d {PROF_RAW}/mfma_{tag} -o pmc -- {b}",
        **{k: f"rocprofv3 --pmc {v} -f csv -d {PROF_RAW}/{k}_{tag} -o pmc -- {b}"
           for k, v in PIPE_COUNTERS.items()},
    }


COPY_COMMANDS = {
    "copy_fetch": f"rocprofv3 --pmc FETCH_SIZE -f csv -d {PROF_RAW}/copy_fetch -o pmc -- "
                  "python3 bench.py --copy-calibration",
    "copy_write": f"rocprofv3 --pmc WRITE_SIZE -f csv -d {PROF_RAW}/copy_write -o pmc -- "
                  "python3 bench.py --copy-calibration",
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the kernel source without comments and blank lines, so that a
    comment edit does not retire counters taken on the same code."""
    with open(KERNEL_SOURCE, "r") as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    code = "\n".join(line.rstrip() for line in src.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------- accounting --

def plan_counts(ids, E_all, shared=0):
    """Rows per expert of one call: ids in [0, E_all - shared) counted; the
    shared expert, if any (the last), gets every token."""
    import numpy as np
    flat = ids.ravel()
    counts = np.bincount(flat[(flat >= 0) & (flat < E_all - shared)], minlength=E_all).astype(np.int64)
    if shared:
        counts[E_all - 1] += ids.shape[0]
    return counts


def algorithmic_work(wl, counts, a16=False, out_bytes=2):
    """Algorithmic bytes / FLOPs of one call from its per-expert row counts.

    Whole path, per expert with n_e > 0 rows: weights 3*Ip*H code bytes +
    FP32 block scales 4*(2*nI*nH + nH*nI); per routed slot 6*Ip*H FLOPs; plus
    the input rows (T*H*2), the output rows (T*H*out_bytes) and the ids and
    weights (8*T*k).  Intermediates (activation codes, h, y) are the
    implementation's and not counted.

    Per launch (the roofline of a single kernel):
      gate_up groups (experts with 1..16 rows: streaming; 17..128: 128-row
        tiles; more: 256-row tiles): weights 2*Ip*H + 8*nI*nH per expert, and
        per slot the activation row (H + 4*nH) read and the h row
        (Ip + 4*nI) written; 4*Ip*H FLOPs per slot;
      down groups (1..16 rows: streaming; more: one launch over the 128- and
        256-row tiles): weights Ip*H + 4*nH*nI per expert, per slot the h row
        (Ip + 4*nI) read and the FP32 y row (4*H) written; 2*Ip*H FLOPs per
        slot;
      combine: per slot 4*H of y read, per token H*out_bytes written and its
        ids and weights.
    """
    import numpy as np
    E, H, I, T, k = wl.E, wl.H, wl.I, wl.T, wl.k
    Ip = 128 * ((I + 127) // 128)
    nH, nI = H // 128, Ip // 128
    counts = np.asarray(counts)
    hit = counts > 0
    P = int(counts.sum())
    w_bytes = int(hit.sum()) * (3 * Ip * H + 4 * (2 * nI * nH + nH * nI))
    path_bytes = w_bytes + T * H * 2 + T * H * out_bytes + 8 * T * k
    path_flops = 6 * P * Ip * H
    groups = {}
    for name, lo, hi in (("stream", 1, 16), ("narrow", 17, 128), ("wide", 129, None)):
        sel = (counts >= lo) & ((counts <= hi) if hi is not None else True)
        rows = int(counts[sel].sum())
        groups[name] = dict(
            experts=int(sel.sum()), rows=rows,
            bytes=int(sel.sum()) * (2 * Ip * H + 8 * nI * nH) + rows * (H + 4 * nH + Ip + 4 * nI),
            flops=4 * rows * Ip * H)
    down = {}
    for name, lo, hi in (("stream", 1, 16), ("wide", 17, None)):
        sel = (counts >= lo) & ((counts <= hi) if hi is not None else True)
        rows = int(counts[sel].sum())
        down[name] = dict(
            experts=int(sel.sum()), rows=rows,
            bytes=int(sel.sum()) * (Ip * H + 4 * nH * nI) + rows * (Ip + 4 * nI + 4 * H),
            flops=2 * rows * Ip * H)
    if a16:
        # W8A16 decode: one gate_up launch over every tile; the activation row
        # is read as BF16 (2H) and h written as BF16 (2Ip), no scales
        rows = int(counts.sum())
        groups = {"decode": dict(experts=int(hit.sum()), rows=rows,
                                 bytes=int(hit.sum()) * (2 * Ip * H + 8 * nI * nH) + rows * (2 * H + 2 * Ip),
                                 flops=4 * rows * Ip * H)}
    combine = dict(experts=0, rows=P, bytes=P * 4 * H + T * H * out_bytes + 8 * T * k, flops=0)
    return dict(path_bytes=path_bytes, path_flops=path_flops, gate_up=groups, down=down, combine=combine,
                experts_hit=int(hit.sum()), slots=P,
                per_expert_gate_up_bytes=2 * Ip * H + 8 * nI * nH)


def add_work(a, b):
    """Sum of two algorithmic_work results (a step of two calls)."""
    if a is None:
        return b
    out = dict(a)
    for key in ("path_bytes", "path_flops", "slots"):
        out[key] = a[key] + b[key]
    out["experts_hit"] = max(a["experts_hit"], b["experts_hit"])
    for grp in ("gate_up", "down"):
        out[grp] = {n: {f: a[grp][n][f] + b[grp][n][f] for f in a[grp][n]} for n in a[grp]}
    out["combine"] = {f: a["combine"][f] + b["combine"][f] for f in a["combine"]}
    return out


def launch_work(work, stage, calls=1):
    """Algorithmic work of one launch timed in library stage `stage` (the
    step's work split evenly over its `calls` calls)."""
    if stage == "combine":
        g = work["combine"]
    elif stage.startswith("gate_up_"):
        g = work["gate_up"]["decode" if "decode" in work["gate_up"] else stage[len("gate_up_"):]]
    else:
        g = work["down"][stage[len("down_"):]]
    return {f: v / calls for f, v in g.items()}


# ------------------------------------------------------------ measurement --

def read_traffic(kernel, tag):
    """HBM bytes per launch of `kernel` from the committed counter summary of
    workload `tag`, or None if absent or taken on different kernel source."""
    path = os.path.join(PROFILES, f"counters_{tag}.md")
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"kernel_source_sha256_16: `([0-9a-f]+)`", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    for line in text.splitlines():
        cells = [c.strip().strip("`") for c in line.split("|")]
        if len(cells) > 5 and cells[1] == kernel:
            try:
                return int(cells[5])
            except ValueError:
                return None
    return None


def roofline(g, stage, launch_ms, peaks, a16=False):
    """The launch against the roof its algorithmic work reaches first."""
    mfma_peak = PEAK_BF16_TFLOPS if a16 else PEAK_FP8_TFLOPS
    t_hbm = g["bytes"] / (PEAK_HBM_GBS * 1e9)
    t_mfma = g["flops"] / (mfma_peak * 1e12)
    if t_mfma >= t_hbm:
        achieved = g["flops"] / (launch_ms * 1e-3) / 1e12
        bound, peak, unit = "mfma", mfma_peak, "TFLOP/s"
        measured = peaks.get("mfma_fp8_TFLOPs") if (peaks and not a16) else None
    else:
        achieved = g["bytes"] / (launch_ms * 1e-3) / 1e9
        bound, peak, unit = "hbm", PEAK_HBM_GBS, "GB/s"
        measured = peaks.get("hbm_read_GBs") if peaks else None
    return {
        "kernel": DESCRIBE["decode_gate_up"] if (a16 and stage.startswith("gate_up")) else DESCRIBE[stage],
        "stage": stage, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
        "frac": achieved / peak, "measured_peak": measured,
        "frac_of_measured": (achieved / measured) if measured else None,
        "traffic": None,
        "algorithmic_bytes_per_launch": int(g["bytes"]), "algorithmic_flops_per_launch": int(g["flops"]),
        "experts_in_launch": g["experts"], "rows_in_launch": g["rows"], "avg_launch_ms": launch_ms,
    }


def path_object(work, ms, peaks, a16=False):
    """The whole step against both peaks (algorithmic bytes and FLOPs); the
    W8A16 decode path's products run on the BF16 MFMA, so its peak is BF16's."""
    mfma_peak = PEAK_BF16_TFLOPS if a16 else PEAK_FP8_TFLOPS
    hbm = work["path_bytes"] / (ms * 1e-3) / 1e9
    mf = work["path_flops"] / (ms * 1e-3) / 1e12
    roof_ms = max(work["path_bytes"] / (PEAK_HBM_GBS * 1e9), work["path_flops"] / (mfma_peak * 1e12)) * 1e3
    o = {"algorithmic_bytes": work["path_bytes"], "algorithmic_flops": work["path_flops"],
         "hbm_GBs": hbm, "hbm_frac": hbm / PEAK_HBM_GBS, "mfma_TFLOPs": mf, "mfma_frac": mf / mfma_peak,
         "mfma_peak_TFLOPs": mfma_peak, "roof_ms": roof_ms, "frac_of_roof": roof_ms / ms,
         "experts_hit": work["experts_hit"]}
    if peaks:
        o["hbm_frac_of_measured"] = hbm / peaks["hbm_read_GBs"]
        if not a16:
            o["mfma_frac_of_measured"] = mf / peaks["mfma_fp8_TFLOPs"]
    return o


def measured_peaks(reps=5):
    """Median of `reps` timed calibration launches of each kind (library
    kernels, see moe_fp8_prefill_calibrate)."""
    import torch

    import fp8_blockwise_routed_amd as pkg
    stream = torch.cuda.current_stream()
    res = {}
    scratch = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    buf = torch.ones(4 << 30, dtype=torch.uint8, device="cuda")
    for kind, n, b, key, scale in ((pkg.MOE_CALIBRATE_MFMA, 20000, scratch, "mfma_fp8_TFLOPs", 1e12),
                                   (pkg.MOE_CALIBRATE_STREAM, 1, buf, "hbm_read_GBs", 1e9)):
        pkg.moe_fp8_prefill_calibrate(kind, n, b, stream)  # first launch untimed
        times, work = [], 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            work = pkg.moe_fp8_prefill_calibrate(kind, n, b, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = sorted(times)[len(times) // 2]
        res[key] = work / (ms * 1e-3) / scale
    del buf, scratch
    torch.cuda.empty_cache()
    res["vendor_mfma_fp8_TFLOPs"] = PEAK_FP8_TFLOPS
    res["vendor_hbm_GBs"] = PEAK_HBM_GBS
    res["how"] = ("median of 5 launches each: eight independent chains of the 16x16x128 FP8 MFMA per wave, "
                  "two waves per SIMD; a streaming read of 4 GiB - 64 KiB with the 16-byte buffer loads and cache "
                  "policy of the GEMMs' weight stream, 16 in flight per thread, 16 waves per CU")
    return res


class Case:
    """One workload on the shared handle: device inputs, the calls of a
    step, and the step's algorithmic work (from the row counts of each call)."""

    def __init__(self, key, wl, x, ids, w, rows_per_call=None):
        import dataclasses

        import numpy as np
        import torch
        self.key, self.wl = key, wl
        self.xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        self.idd = torch.from_numpy(ids).cuda()
        self.wd = torch.from_numpy(w).cuda()
        self.out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
        rpc = rows_per_call or wl.T
        self.calls = [(a, min(a + rpc, wl.T)) for a in range(0, wl.T, rpc)]
        self.work = None
        for a, b in self.calls:
            part = dataclasses.replace(wl, T=b - a)
            self.work = add_work(self.work, algorithmic_work(part, plan_counts(ids[a:b], wl.E + wl.shared,
                                                                               wl.shared)))


def run_case(moe, case, args, peaks, stream, step_fn=None, a16=False):
    """Warmup, stage breakdown, timed steps and the protocol for one case."""
    import torch

    import fp8_blockwise_routed_amd as pkg
    wl = case.wl
    n_calls = len(case.calls)

    def step():
        if step_fn is not None:
            return step_fn()
        for a, b in case.calls:
            fn = pkg.moe_fp8_prefill_run_decode if a16 else pkg.moe_fp8_prefill_run
            rc = fn(moe.handle, case.xd[a:b], case.idd[a:b], case.wd[a:b], b - a, case.out[a:b], stream)
            if rc != pkg.MOE_OK:
                raise pkg.MoeError(rc, "run")

    log(f"[bench] {case.key}: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    res = {"workload": wl.name, "rows": wl.T, "calls_per_step": n_calls}
    timing = not args.no_timing_events
    stage = None
    if timing:
        pkg.moe_fp8_prefill_set_timing(moe.handle, True)
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        stages = pkg.moe_fp8_prefill_read_timing(moe.handle)
        passes = stages.shape[0] // 5  # passes per step
        per_step = stages[: 5 * passes].reshape(5, passes, stages.shape[1]).sum(axis=1).mean(axis=0)
        res["stages_ms"] = {name: float(v) for name, v in zip(pkg.STAGES, per_step)}
        candidates = ["gate_up_stream", "gate_up_narrow", "gate_up_wide", "down_stream", "down_wide", "combine"]
        stage = max(candidates, key=lambda s: res["stages_ms"][s])
        pkg.moe_fp8_prefill_set_timing_stages(moe.handle, [stage])
    log(f"[bench] {case.key}: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    live = pkg.moe_fp8_prefill_read_timing(moe.handle) if timing else None
    pkg.moe_fp8_prefill_set_timing(moe.handle, False)
    if moe.status() != pkg.MOE_OK:
        raise RuntimeError("device reported an error")
    ms = elapsed * 1e3 / args.steps
    res["ms_per_step"] = ms
    res["tokens_per_s"] = wl.T * args.steps / elapsed
    res["path"] = path_object(case.work, ms, peaks, a16=a16)
    if stage is not None and live is not None and len(live):
        launch_ms = float(live[:, pkg.STAGES.index(stage)].mean())
        passes = max(1, live.shape[0] // max(1, args.steps))
        res["roofline"] = roofline(launch_work(case.work, stage, passes), stage, launch_ms, peaks, a16=a16)

    if args.protocol_calls > 0:
        log(f"[bench] {case.key}: protocol, {args.protocol_calls} calls with a MALL flush before each")
        flush = torch.empty(MALL_FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        times, same, ref = [], 0, None
        for i in range(args.protocol_calls):
            flush.fill_(i & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
            if ref is None:
                ref = case.out.clone()
                same += 1
            else:
                same += int(torch.equal(case.out, ref))
        del flush
        times.sort()
        med = times[len(times) // 2]
        digest = hashlib.sha256(ref.view(torch.int16).cpu().numpy().tobytes()).hexdigest()[:16]
        res["protocol"] = {
            "calls": args.protocol_calls, "median_ms": med, "p10_ms": times[len(times) // 10],
            "p90_ms": times[(9 * len(times)) // 10], "median_tokens_per_s": wl.T / (med * 1e-3),
            "mall_flush_bytes": MALL_FLUSH_BYTES, "outputs_identical": f"{same}/{args.protocol_calls}",
            "output_sha256_16": digest,
        }
        if same != args.protocol_calls:
            raise RuntimeError(f"{case.key}: the outputs of the protocol calls differ")
    return res


def cpu_baseline(layer, wl, x, ids, w, n_tokens, repeats, a16=False):
    """The oracle, as it stands, on the first n_tokens rows of the same batch:
    median wall clock of `repeats` runs."""
    import numpy as np

    import oracle
    ids, w = ids[:n_tokens], w[:n_tokens]
    if wl.shared:  # the shared expert's slot, id E and weight 1, last
        ids = np.concatenate([ids, np.full((n_tokens, 1), wl.E, np.int32)], axis=1)
        w = np.concatenate([w, np.ones((n_tokens, 1), np.float32)], axis=1)
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        oracle.forward(layer, x[:n_tokens], ids, w, wl.rho, oracle.OUT_BF16, n_shared=wl.shared, a16=a16)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    return dict(value=n_tokens / dt, unit="tokens/s", cores=oracle.max_threads(), cpu_model=cpu_model(),
                kind="oracle",
                sample=f"first {n_tokens} of the {wl.T} rows of {wl.name} with all their routed experts"
                       f"{' (W8A16 form)' if a16 else ''}; median of {repeats} runs, {dt:.2f} s each")


# --------------------------------------------------------------- profiles --

def _csv_rows(pattern):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(pattern, recursive=True)):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _base_name(name):
    """Kernel base name from a demangled rocprofv3 kernel name."""
    name = name.split("(")[0].replace("void ", "").strip()
    name = name.split("<")[0]
    return name.split("::")[-1]


def _per_kernel(rows, counter):
    """Mean value of `counter` per dispatch, by kernel base name."""
    acc = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        acc.setdefault(_base_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def summarize_profiles(out_dir: str) -> int:
    """Write the committed profile summaries from the rocprofv3 CSV output
    under out_dir (the runs printed by --print-profile-commands)."""
    src = kernel_source_hash()
    os.makedirs(PROFILES, exist_ok=True)
    wrote = 0
    copy_f = _per_kernel(_csv_rows(os.path.join(out_dir, "copy_fetch", "**", "*counter_collection.csv")),
                         "FETCH_SIZE")
    copy_w = _per_kernel(_csv_rows(os.path.join(out_dir, "copy_write", "**", "*counter_collection.csv")),
                         "WRITE_SIZE")
    cf = next((v[0] for k, v in copy_f.items() if "copy" in k.lower()), None)
    cw = next((v[0] for k, v in copy_w.items() if "copy" in k.lower()), None)
    copy_kib = (1 << 30) / 1024
    for tag in PROFILED:
        cmds = profile_commands(tag)
        stats = _csv_rows(os.path.join(out_dir, f"kt_{tag}", "**", "*kernel_stats.csv"))
        trace = _csv_rows(os.path.join(out_dir, f"kt_{tag}", "**", "*kernel_trace.csv"))
        per = {}
        for r in trace:
            per.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        durations = {}
        if stats:
            lines = [f"# Kernel time, {TITLES[tag]}", "", "Command (repository root, one MI355X):", "",
                     f"    {cmds['trace']}", "", f"- kernel_source_sha256_16: `{src}`", "",
                     "Average, min and max are rocprofv3's --stats over every dispatch; the median is over the "
                     "same dispatches in the kernel trace.", "",
                     "| kernel | calls | average us | median us | min us | max us | % of GPU time |",
                     "|---|---|---|---|---|---|---|"]
            for r in stats:
                d = sorted(per.get(r["Name"], []))
                med = d[len(d) // 2] / 1e3 if d else float("nan")
                lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {med:.1f} | "
                             f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                             f"{float(r['Percentage']):.2f} |")
                durations[_base_name(r["Name"])] = med * 1e3 if d else float(r["AverageNs"])
            lines += ["", "The layout kernels run once, inside create(), outside the timed steps."]
            with open(os.path.join(PROFILES, f"kernel_stats_{tag}.md"), "w") as f:
                f.write("\n".join(lines) + "\n")
            wrote += 1
        fetch = _per_kernel(_csv_rows(os.path.join(out_dir, f"fetch_{tag}", "**", "*counter_collection.csv")),
                            "FETCH_SIZE")
        write = _per_kernel(_csv_rows(os.path.join(out_dir, f"write_{tag}", "**", "*counter_collection.csv")),
                            "WRITE_SIZE")
        if fetch and write and cf and cw:
            fs, ws = copy_kib / cf, copy_kib / cw
            lines = [f"# HBM traffic per launch, {TITLES[tag]}", "",
                     "Commands (repository root, one MI355X), one counter per run:", "",
                     f"    {cmds['fetch']}", f"    {cmds['write']}",
                     f"    {COPY_COMMANDS['copy_fetch']}", f"    {COPY_COMMANDS['copy_write']}", "",
                     "Counters are KiB per dispatch, averaged over each kernel's dispatches.  The copy runs "
                     "move 1 GiB (1048576 KiB) each way with torch's device copy; their readings give the "
                     f"scale factors FETCH_SIZE x {fs:.4f} and WRITE_SIZE x {ws:.4f}.", "",
                     f"- copy_FETCH_SIZE_kib: {cf:.1f}", f"- copy_WRITE_SIZE_kib: {cw:.1f}",
                     f"- kernel_source_sha256_16: `{src}`", "",
                     "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch |",
                     "|---|---|---|---|---|"]
            for k in sorted(fetch):
                if k not in write:
                    continue
                hbm = int(round((fetch[k][0] * fs + write[k][0] * ws) * 1024))
                lines.append(f"| `{k}` | {fetch[k][1]} | {fetch[k][0]:.1f} | {write[k][0]:.1f} | {hbm} |")
            with open(os.path.join(PROFILES, f"counters_{tag}.md"), "w") as f:
                f.write("\n".join(lines) + "\n")
            wrote += 1
        mrows = _csv_rows(os.path.join(out_dir, f"mfma_{tag}", "**", "*counter_collection.csv"))
        if mrows:
            busy = _per_kernel(mrows, "SQ_VALU_MFMA_BUSY_CYCLES")
            mops = _per_kernel(mrows, "SQ_INSTS_VALU_MFMA_MOPS_F8")
            gui = _per_kernel(mrows, "GRBM_GUI_ACTIVE")
            simds, xccs = 1024, 8  # 256 CUs x 4 SIMDs, in 8 XCDs
            lines = [f"# Matrix-core counters per launch, {TITLES[tag]}", "",
                     "Command (repository root, one MI355X):", "", f"    {cmds['mfma']}", "",
                     "rocprofv3 sums each counter over its dimensions: SQ_VALU_MFMA_BUSY_CYCLES over every SIMD, "
                     f"GRBM_GUI_ACTIVE over the {xccs} XCDs, so one XCD's active cycles are GRBM_GUI_ACTIVE / "
                     f"{xccs}.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {xccs} x {simds} SIMDs).  "
                     "SQ_INSTS_VALU_MFMA_MOPS_F8 counts FP8 MFMA operations / 512 (padded rows of a 16-row "
                     "subtile included).  The clock is one XCD's active cycles over the kernel's median duration "
                     "in the trace run of the same workload (kernel_stats file).  Launches that find no work (an "
                     "empty tile list) are left out.", "",
                     f"- kernel_source_sha256_16: `{src}`", "",
                     "| kernel | dispatches | MFMA busy | FP8 TFLOP per launch | GRBM_GUI_ACTIVE cycles (sum) | "
                     "clock GHz | FP8 TFLOP/s |", "|---|---|---|---|---|---|---|"]
            for k in sorted(busy):
                if k not in gui or not (k.startswith("gate_up") or k.startswith("down") or k.startswith("tie")):
                    continue
                if mops.get(k, (0.0, 0))[0] == 0.0:
                    continue
                cyc = gui[k][0] / xccs
                util = busy[k][0] / (cyc * simds) if cyc else float("nan")
                tflop = mops[k][0] * 512 / 1e12 if k in mops else float("nan")
                dur = durations.get(k)
                ghz = cyc / dur if dur else float("nan")
                rate = tflop / (dur * 1e-9) if dur else float("nan")
                lines.append(f"| `{k}` | {busy[k][1]} | {util:.3f} | {tflop:.4f} | {gui[k][0]:.0f} | "
                             f"{ghz:.2f} | {rate:.0f} |")
            with open(os.path.join(PROFILES, f"mfma_{tag}.md"), "w") as f:
                f.write("\n".join(lines) + "\n")
            wrote += 1
        wrote += _pipe_summary(out_dir, tag, cmds, src)
    log(f"[bench] wrote {wrote} summaries")
    return 0 if wrote else 1


def _pipe_summary(out_dir, tag, cmds, src):
    """profiles/pipe_<tag>.md from the three pipe_* counter passes."""
    vals = {}
    for k in PIPE_COUNTERS:
        rows = _csv_rows(os.path.join(out_dir, f"{k}_{tag}", "**", "*counter_collection.csv"))
        if not rows:
            return 0
        names = {r["Counter_Name"] for r in rows}
        for c in names:
            for kern, (v, _n) in _per_kernel(rows, c).items():
                vals.setdefault(kern, {})[c if c != "GRBM_GUI_ACTIVE" else f"GUI_{k}"] = v
    cus, simds, xccs = 256, 1024, 8
    lines = [f"# Where the cycles go, {TITLES[tag]}", "", "Commands (repository root, one MI355X), one pass each:", ""]
    lines += [f"    {cmds[k]}" for k in PIPE_COUNTERS]
    lines += ["", "Per launch, averaged over its dispatches.  C = one XCD's active cycles (GRBM_GUI_ACTIVE / "
              f"{xccs}, from the same pass).  The SQ counts wave time in its own units, so the wave-time "
              "fractions divide by SQ_WAVE_CYCLES: waiting = SQ_WAIT_INST_ANY (a wave stopped at a wait for "
              "its own loads, LDS reads or stores), valu / lds / vmem = SQ_ACTIVE_INST_* (issuing that kind).  "
              f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (C x {simds} SIMDs).  Per-CU unit busy = counter / "
              f"(C x {cus} CUs): TA (address unit), TD (data return to VGPRs and LDS), LDS (SQ_LDS_IDX_ACTIVE); "
              "TD stalled on TC = TD_TC_STALL / (C x 256).  L2 read latency = TCP_TCC_READ_REQ_LATENCY / "
              "TCP_TCC_READ_REQ, in cycles.", "", f"- kernel_source_sha256_16: `{src}`", "",
              "| kernel | MFMA busy | waiting | valu | lds | vmem | LDS busy | bank conflicts / LDS instr | "
              "TA busy | TD busy | TD stalled on TC | L2 read latency | VALU instr / MFMA |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(vals):
        v = vals[k]
        if not (k.startswith("gate_up") or k.startswith("down") or k.startswith("combine")):
            continue
        if v.get("SQ_INSTS_VMEM_RD", 0.0) == 0.0:
            continue  # a launch that found no work
        ca = v["GUI_pipe_a"] / xccs
        cb = v["GUI_pipe_b"] / xccs
        wave = v["SQ_WAVE_CYCLES"] or float("nan")
        lds_i = v.get("SQ_INSTS_LDS", 0.0)
        mf = v.get("SQ_INSTS_MFMA", 0.0)
        row = [v["SQ_VALU_MFMA_BUSY_CYCLES"] / (cb * simds), v["SQ_WAIT_INST_ANY"] / wave,
               v["SQ_ACTIVE_INST_VALU"] / wave, v["SQ_ACTIVE_INST_LDS"] / wave, v["SQ_ACTIVE_INST_VMEM"] / wave,
               v["SQ_LDS_IDX_ACTIVE"] / (cb * cus), (v["SQ_LDS_BANK_CONFLICT"] / lds_i) if lds_i else 0.0,
               v["TA_TA_BUSY"] / (cb * cus), v["TD_TD_BUSY"] / (cb * cus), v["TD_TC_STALL"] / (cb * cus)]
        lat = v["TCP_TCC_READ_REQ_LATENCY"] / v["TCP_TCC_READ_REQ"] if v.get("TCP_TCC_READ_REQ") else float("nan")
        ratio = (v["SQ_INSTS_VALU"] - mf) / mf if mf else float("nan")
        lines.append(f"| `{k}` | " + " | ".join(f"{x:.3f}" for x in row) + f" | {lat:.0f} | {ratio:.1f} |")
    lines += ["", "Unit busy counters count a cycle in which the unit holds any work, waiting included, so "
              "they bound the unit's share from above rather than measure its throughput."]
    with open(os.path.join(PROFILES, f"pipe_{tag}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    return 1


# ------------------------------------------------------------------- main --

def streamed_bench(args, wl, layer, xd, idd, wd, out) -> int:
    """Whole-model prefill through `L` layers whose weights are copied from
    page-locked host memory into two device slots ("ktransformers #2244",
    Design: one reusable per-layer slot refilled from the host): the copy of
    layer i+1 (copy stream) overlaps the pass of layer i (compute stream).
    Every layer stages the same host arrays (a repeated slot), so each pass
    transfers the full slot."""
    import torch

    import fp8_blockwise_routed_amd as pkg
    import gen
    L = args.streamed_layers
    log("[bench] pinning the host copy of the layer")
    host = {}
    for name in ("gate", "up", "down", "gate_scale", "up_scale", "down_scale"):
        a = getattr(layer, name)
        t = torch.empty(a.shape, dtype=torch.uint8 if a.dtype.itemsize == 1 else torch.float32,
                        pin_memory=True)
        t.numpy()[...] = a
        host[name] = t
    hl = gen.Layer(layer.E, layer.H, layer.I, *(host[n] for n in ("gate", "up", "down", "gate_scale",
                                                                 "up_scale", "down_scale")))
    slot_bytes = sum(int(t.numel() * t.element_size()) for t in host.values())
    sm = pkg.StreamedMoeFp8Prefill(layer, wl.k, n_slots=2, routed_scale=wl.rho, max_rows=8192,
                                   out_dtype=pkg.MOE_DTYPE_BF16, shared_experts=wl.shared)
    copy = torch.cuda.Stream()
    comp = torch.cuda.current_stream()

    def model(n):
        sm.stage(0, hl, stream=copy)
        for i in range(n):
            if i + 1 < n:
                sm.stage((i + 1) % 2, hl, stream=copy)
            sm.select(i % 2)
            sm.run(xd, idd, wd, out=out, stream=comp)

    log("[bench] warmup (2 layers)")
    model(2)
    torch.cuda.synchronize()
    log(f"[bench] timing {L} layers")
    t0 = time.perf_counter()
    model(L)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if sm.status() != pkg.MOE_OK:
        raise RuntimeError("device reported an error")
    sm.close()
    print(json.dumps(streamed_result(wl, L, slot_bytes, elapsed)), flush=True)
    return 0


def streamed_result(wl, L, slot_bytes, elapsed):
    """The JSON object of a streamed-layer run: L layers in `elapsed` seconds,
    each staging `slot_bytes` from the host (W8A8 prefill passes)."""
    return {
        "metric": "whole-model prefill input tokens/sec through streamed layer slots (1 MI355X, "
                  "host-link bound)",
        "value": wl.T / elapsed, "unit": "tokens/s", "n_gpus": 1, "steps": L, "warmup": 2,
        "ms_per_step": elapsed * 1e3 / L, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "slots": 2, "slot_bytes": slot_bytes,
                   "host_memory": "page-locked, one layer staged L times"},
        "h2d_GBs": L * slot_bytes / elapsed / 1e9,
        "per_layer_tokens_s": wl.T * L / elapsed,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default=None,
                    help="time this workload alone (default: the T=8192 Zipf headline, then the 2x4096, "
                         "T=4096 and T=256 sub-objects on the same layer)")
    ap.add_argument("--protocol-calls", type=int, default=32,
                    help="calls of the per-call protocol (events, MALL flush, output comparison); 0 skips it")
    ap.add_argument("--cpu-tokens", type=int, default=256,
                    help="rows of the headline batch the CPU oracle is timed on (0 skips it)")
    ap.add_argument("--cpu-repeats", type=int, default=3)
    ap.add_argument("--no-timing-events", action="store_true",
                    help="skip the per-launch HIP events (roofline needs them)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak calibration")
    ap.add_argument("--peaks", action="store_true", help="only the measured-peak calibration")
    ap.add_argument("--streamed-layers", type=int, default=0, metavar="L",
                    help="instead: whole-model prefill through L layers staged from pinned host memory "
                         "into two device slots (double-buffered H2D overlapped with compute)")
    ap.add_argument("--decode", type=int, default=0, metavar="T",
                    help="time the W8A16 decode path (run_decode) on the first T rows of the workload's "
                         "batch instead of the W8A8 prefill path")
    ap.add_argument("--rows", type=int, default=0, metavar="T",
                    help="the chosen workload's layer and routing recipe with T rows instead (one call "
                         "up to 8192 rows, passes of 8192 above)")
    ap.add_argument("--router", action="store_true",
                    help="start each step from FP32 router logits (run_logits: on-device top-k router, then "
                         "the path) instead of given ids and weights")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries from rocprofv3 CSV output under DIR")
    ap.add_argument("--print-profile-commands", action="store_true",
                    help="print the rocprofv3 commands whose output --summarize-profiles reads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the reference for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.summarize_profiles:
        return summarize_profiles(args.summarize_profiles)
    if args.print_profile_commands:
        for tag in PROFILED:
            for cmd in profile_commands(tag).values():
                print(cmd)
        for cmd in COPY_COMMANDS.values():
            print(cmd)
        return 0
    if args.gpus != 1:
        print(json.dumps({"error": "this path runs on one GPU; multi-GPU sharding is design only "
                                   "(expert-parallel all-to-all), so --gpus must be 1"}))
        return 2
    if args.copy_calibration:
        import torch
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n}))
        return 0

    import dataclasses

    import torch

    import fp8_blockwise_routed_amd as pkg
    import gen

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    peaks = None if args.no_peaks else measured_peaks()
    if args.peaks:
        print(json.dumps({"measured_peaks": peaks}), flush=True)
        return 0

    wl = gen.WORKLOADS[args.workload or HEADLINE]
    if args.rows > 0:
        base = wl.name.rsplit("_t", 1)[0] if "_t" in wl.name else wl.name
        suffix = wl.name.rsplit("_t", 1)[1].lstrip("0123456789") if "_t" in wl.name else ""
        wl = dataclasses.replace(wl, T=args.rows, name=f"{base}_t{args.rows}{suffix}")
    log(f"[bench] generating {wl.name}")
    t0 = time.perf_counter()
    layer = gen.make_layer(wl.E + wl.shared, wl.H, wl.I, seed=wl.seed)
    x, ids, w, _ = gen.make_inputs(wl)
    a16 = args.decode > 0
    if a16:  # the first T rows of the batch through the W8A16 decode path
        Td = min(args.decode, wl.T)
        x, ids, w = x[:Td], ids[:Td], w[:Td]
        wl = dataclasses.replace(wl, T=Td, name=f"{wl.name}_decode_t{Td}")
    log(f"[bench] generated in {time.perf_counter() - t0:.1f} s; creating the handle")
    moe = pkg.MoeFp8Prefill(layer, wl.k, routed_scale=wl.rho, max_rows=8192,
                            out_dtype=pkg.MOE_DTYPE_BF16, shared_experts=wl.shared)
    head = Case("headline", wl, x, ids, w)
    if args.streamed_layers > 0:
        moe.close()
        return streamed_bench(args, wl, layer, head.xd, head.idd, head.wd, head.out)

    step_fn = None
    if args.router:
        router = pkg.MOE_ROUTER_SOFTMAX if wl.route == gen.ROUTE_SOFTMAX else pkg.MOE_ROUTER_SIGMOID
        ld = torch.from_numpy(gen.make_logits(wl.T, wl.E, wl.route, wl.seed, wl.n_masked)).cuda()

        def step_fn():
            rc = pkg.moe_fp8_prefill_run_logits(moe.handle, head.xd, ld, router, wl.T, head.out, stream)
            if rc != pkg.MOE_OK:
                raise pkg.MoeError(rc, "run_logits")

    h = run_case(moe, head, args, peaks, stream, step_fn=step_fn, a16=a16)
    res = {
        "metric": METRIC, "value": h["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": h["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 x fp8_e4m3 (fp32 accumulate)" if a16 else "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": wl.name + ("" if a16 else " (one call)"), "experts": wl.E, "top_k": wl.k,
                   "hidden": wl.H, "intermediate": wl.I, "rows": wl.T, "routed_scale": wl.rho,
                   "outlier_rows": wl.outlier_frac, "masked_experts": wl.n_masked, "seed": wl.seed,
                   "shared_experts": wl.shared, "path": "decode (W8A16)" if a16 else "prefill (W8A8)",
                   "input": "router logits" if args.router else "top-k ids and weights"},
    }
    for key in ("path", "roofline", "stages_ms", "protocol"):
        if key in h:
            res[key] = h[key]
    tag = next((t for t, name in PROFILED.items() if name == wl.name), None)
    if "roofline" in res and tag and not a16:
        res["roofline"]["traffic"] = read_traffic(KERNELS[res["roofline"]["stage"]], tag)
    if peaks:
        res["measured_peaks"] = peaks

    if args.router:
        ids_r = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
        w_r = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 50
        e0.record(stream)
        for _ in range(reps):
            pkg.moe_fp8_prefill_route(moe.handle, ld, router, wl.T, ids_r, w_r, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        r_us = e0.elapsed_time(e1) * 1e3 / reps
        r_bytes = wl.T * wl.E * 4 + wl.T * wl.k * 8
        res["router"] = {"kernel": "route_kernel", "kind": "softmax" if router == 0 else "sigmoid",
                         "avg_launch_us": r_us, "algorithmic_bytes": r_bytes, "GBs": r_bytes / (r_us * 1e-6) / 1e9,
                         "ids_equal_given": bool(torch.equal(ids_r, head.idd))}

    if args.workload is None and args.rows == 0 and not a16 and not args.router:
        subs = {}
        for key, name, rpc in SUBS:
            swl = gen.WORKLOADS[name]
            sx, sids, sw, _ = gen.make_inputs(swl)
            case = Case(key, swl, sx, sids, sw, rows_per_call=rpc)
            r = run_case(moe, case, args, peaks, stream)
            stag = next((t for t, n in PROFILED.items() if n == name), None)
            if "roofline" in r and stag and rpc is None:
                r["roofline"]["traffic"] = read_traffic(KERNELS[r["roofline"]["stage"]], stag)
            if rpc is not None:
                r["workload"] = f"{name} ({swl.T // rpc} calls of {rpc} rows)"
                # the same rows as the headline's one call: equal bit for bit
                r["equals_one_call"] = bool(torch.equal(case.out, head.out))
            subs[key] = r
            del case
        res["workloads"] = subs

    if args.cpu_tokens > 0:
        log(f"[bench] CPU oracle on {args.cpu_tokens} rows")
        res["cpu_baseline"] = cpu_baseline(layer, wl, x, ids, w, min(args.cpu_tokens, wl.T),
                                           a16=a16, repeats=max(1, args.cpu_repeats))
    moe.close()
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
