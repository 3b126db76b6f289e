#!/usr/bin/env python3
"""Benchmark: input tokens/s of the routed-expert FP8 MoE prefill layer on one
MI355X, with the dominant kernel's roofline and the CPU oracle beside it.

A step is one call of the whole path (plan, quantise, gate_up, down, combine)
on one batch of seeded synthetic input already resident in HBM.  Default
workload: the GLM-class layer (E=256, top-8, H=6144, I=2048, 9.002 GiB of FP8
weights and FP32 block scales) at T=256 rows, sigmoid top-8 routing with
routed scale 2.5 and 1% outlier rows x100.

Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense BF16 MFMA, TFLOP/s (the W8A16 decode path)
METRIC = "input tokens/sec per MoE layer (1 MI355X) + % FP8 MFMA peak / % HBM peak"
PROFILES = os.path.join(ROOT, "profiles")
COUNTERS_MD = os.path.join(PROFILES, "gate_up_stream_glm_e256_t256_counters.md")
GATE_UP_KERNELS = {
    "stream": "gate_up_stream_kernel (experts with 1..16 rows)",
    "narrow": "gate_up_narrow_kernel (experts with 17..128 rows)",
    "wide": "gate_up_wide_kernel (experts with more than 128 rows)",
    "decode": "gate_up_a16_kernel (W8A16 decode, every expert hit)",
}


def gate_up_stage(kind):
    """The library's timing stage of a gate_up launch group (the W8A16
    decode path's single gate_up launch is timed in the streaming slot)."""
    return "gate_up_stream" if kind == "decode" else "gate_up_" + kind
STATS_MD = os.path.join(PROFILES, "kernel_stats_glm_e256_t256.md")
KERNEL_SOURCE = os.path.join(ROOT, "fp8_blockwise_routed_amd", "csrc", "moe_kernels.hip")
DOMINANT = "gate_up_stream_kernel"   # the 1-subtile gate_up launch (experts with 1..16 rows)

# The commands whose output --summarize-profiles reads (run from the repository root).
PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_kt -o kt -- "
             "python3 bench.py --steps 10 --warmup 3 --cpu-tokens 0",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/prof_fetch -o fetch -- "
             "python3 bench.py --steps 3 --warmup 1 --cpu-tokens 0",
    "write": "rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/prof_write -o write -- "
             "python3 bench.py --steps 3 --warmup 1 --cpu-tokens 0",
    "copy_fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/prof_copy_fetch -o cf -- "
                  "python3 bench.py --copy-calibration",
    "copy_write": "rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/prof_copy_write -o cw -- "
                  "python3 bench.py --copy-calibration",
    "trace_zipf": "rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_kt_zipf -o kt -- "
                  "python3 bench.py --workload glm_e256_k8_h6144_i2048_t8192_zipf --steps 5 "
                  "--warmup 2 --cpu-tokens 0",
    "trace_probe": "rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_kt_probe -o kt -- "
                   "python3 bench.py --workload probe_e8_k8_h6144_i2048_t4096 --steps 5 "
                   "--warmup 2 --cpu-tokens 0",
    "trace_router": "rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_kt_router -o kt -- "
                    "python3 bench.py --workload glm_e256_k8_h6144_i2048_t4096_uniform --router "
                    "--steps 5 --warmup 2 --cpu-tokens 0",
}

# Extra kernel-time summaries: (command key, output dir, summary file, title).
EXTRA_TRACES = [
    ("trace_zipf", "prof_kt_zipf", "kernel_stats_glm_e256_t8192_zipf.md",
     "GLM-class layer E=256 top-8 H=6144 I=2048, T=8192 rows, Zipf(1.2) routing, one pass"),
    ("trace_probe", "prof_kt_probe", "kernel_stats_probe_e8_t4096.md",
     "compute-bound probe: E=8, every token to all 8 experts, H=6144 I=2048, T=4096"),
    ("trace_router", "prof_kt_router", "kernel_stats_glm_e256_t4096_router.md",
     "GLM-class layer E=256 top-8, T=4096 rows from router logits (route_kernel + path)"),
]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the kernel source without comments and blank lines, so that a
    comment edit does not retire counters taken on the same code."""
    import re
    with open(KERNEL_SOURCE, "r") as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    code = "\n".join(line.rstrip() for line in src.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def algorithmic_work(wl, counts, a16=False):
    """Algorithmic bytes / FLOPs from the plan's per-expert row counts.

    Per expert with n_e > 0 rows: weights 3*Ip*H code bytes + FP32 block
    scales 4*(2*nI*nH + nH*nI); per routed slot: 6*Ip*H FLOPs.  Plus the
    input rows (T*H*2) and output rows (T*H*2 for BF16) and ids/weights (8*P).
    Returns the whole path and, for each gate_up launch (experts with 1..16
    rows: streaming; 17..128: 128-row tiles; more: 256-row tiles), its
    weights 2*Ip*H + 8*nI*nH per expert, the activation row (H + 4*nH) read
    and the h row (Ip + 4*nI) written per slot, and 4*Ip*H FLOPs per slot.
    """
    import numpy as np
    E, H, I, T, k = wl.E, wl.H, wl.I, wl.T, wl.k
    Ip = 128 * ((I + 127) // 128)
    nH, nI = H // 128, Ip // 128
    hit = counts > 0
    P = int(counts.sum())
    w_bytes = int(hit.sum()) * (3 * Ip * H + 4 * (2 * nI * nH + nH * nI))
    path_bytes = w_bytes + T * H * 2 + T * H * 2 + 8 * T * k
    path_flops = 6 * P * Ip * H
    groups = {}
    for name, lo, hi in (("stream", 1, 16), ("narrow", 17, 128), ("wide", 129, None)):
        sel = (counts >= lo) & ((counts <= hi) if hi is not None else True)
        rows = int(counts[sel].sum())
        groups[name] = dict(
            experts=int(sel.sum()), rows=rows,
            bytes=int(sel.sum()) * (2 * Ip * H + 8 * nI * nH) + rows * (H + 4 * nH + Ip + 4 * nI),
            flops=4 * rows * Ip * H)
    if a16:
        # W8A16 decode: one gate_up launch over every tile; the activation row
        # is read as BF16 (2H) and h written as BF16 (2Ip), no scales
        rows = int(counts.sum())
        groups = {"decode": dict(experts=int(hit.sum()), rows=rows,
                                 bytes=int(hit.sum()) * (2 * Ip * H + 8 * nI * nH) + rows * (2 * H + 2 * Ip),
                                 flops=4 * rows * Ip * H)}
    return dict(path_bytes=path_bytes, path_flops=path_flops, gate_up=groups,
                experts_hit=int(hit.sum()), slots=P,
                per_expert_gate_up_bytes=2 * Ip * H + 8 * nI * nH)


def read_traffic():
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, or None if absent or taken on different kernel source."""
    fields = {}
    try:
        with open(COUNTERS_MD) as f:
            for line in f:
                if line.startswith("- ") and ": " in line:
                    key, val = line[2:].split(": ", 1)
                    fields[key.strip()] = val.strip().strip("`")
    except OSError:
        return None
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _csv_rows(pattern):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(pattern, recursive=True)):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _mean_counter(rows, name_part, counter):
    vals = [float(r["Counter_Value"]) for r in rows
            if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def summarize_profiles(out_dir: str) -> int:
    """Write the committed profile summaries from rocprofv3 CSV output under
    out_dir (the PROFILE_COMMANDS runs)."""
    stats = _csv_rows(os.path.join(out_dir, "prof_kt", "**", "*kernel_stats.csv"))
    if not stats:
        log("no kernel_stats.csv found")
        return 1
    src = kernel_source_hash()
    lines = ["# Kernel time, GLM-class layer E=256 top-8 H=6144 I=2048, T=256 rows", "",
             "Command (repository root, one MI355X):", "", f"    {PROFILE_COMMANDS['trace']}", "",
             f"- kernel_source_sha256_16: `{src}`", "",
             "| kernel | calls | average us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.2f} |")
    lines += ["", "The layout kernels run once, inside create() (weight upload), outside the timed steps."]
    os.makedirs(PROFILES, exist_ok=True)
    with open(STATS_MD, "w") as f:
        f.write("\n".join(lines) + "\n")
    for key, sub, md, title in EXTRA_TRACES:
        rows = _csv_rows(os.path.join(out_dir, sub, "**", "*kernel_stats.csv"))
        if not rows:
            continue
        lines = [f"# Kernel time, {title}", "",
                 "Command (repository root, one MI355X):", "", f"    {PROFILE_COMMANDS[key]}", "",
                 f"- kernel_source_sha256_16: `{src}`", "",
                 "| kernel | calls | average us | min us | max us | % of GPU time |",
                 "|---|---|---|---|---|---|"]
        for r in rows:
            lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                         f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                         f"{float(r['Percentage']):.2f} |")
        lines += ["", "The layout kernels run once, inside create(), outside the timed steps."]
        with open(os.path.join(PROFILES, md), "w") as f:
            f.write("\n".join(lines) + "\n")

    fetch = _csv_rows(os.path.join(out_dir, "prof_fetch", "**", "*counter_collection.csv"))
    write = _csv_rows(os.path.join(out_dir, "prof_write", "**", "*counter_collection.csv"))
    cfetch = _csv_rows(os.path.join(out_dir, "prof_copy_fetch", "**", "*counter_collection.csv"))
    cwrite = _csv_rows(os.path.join(out_dir, "prof_copy_write", "**", "*counter_collection.csv"))
    f_kib, nf = _mean_counter(fetch, DOMINANT, "FETCH_SIZE")
    w_kib, nw = _mean_counter(write, DOMINANT, "WRITE_SIZE")
    cf_kib, _ = _mean_counter(cfetch, "copyBuffer", "FETCH_SIZE")
    cw_kib, _ = _mean_counter(cwrite, "copyBuffer", "WRITE_SIZE")
    if None in (f_kib, w_kib, cf_kib, cw_kib):
        log("counter CSVs incomplete")
        return 1
    copy_kib = (1 << 30) / 1024
    f_scale, w_scale = copy_kib / cf_kib, copy_kib / cw_kib
    hbm = int(round((f_kib * f_scale + w_kib * w_scale) * 1024))
    lines = [f"# HBM traffic of {DOMINANT}<5> (gate_up, experts with 1..16 rows), "
             "GLM-class layer E=256 T=256", "",
             "Commands (repository root, one MI355X), one counter per run:", ""]
    lines += [f"    {PROFILE_COMMANDS[k]}" for k in ("fetch", "write", "copy_fetch", "copy_write")]
    lines += ["", "Counters are KiB per dispatch, averaged over the kernel's dispatches "
                  f"({nf} FETCH, {nw} WRITE).  The copy runs move 1 GiB (1048576 KiB) each way "
                  "with torch's device copy; its readings give the scale factors.", "",
              f"- FETCH_SIZE_kib_per_dispatch: {f_kib:.1f}",
              f"- WRITE_SIZE_kib_per_dispatch: {w_kib:.1f}",
              f"- copy_FETCH_SIZE_kib: {cf_kib:.1f}",
              f"- copy_WRITE_SIZE_kib: {cw_kib:.1f}",
              f"- fetch_scale: {f_scale:.4f}",
              f"- write_scale: {w_scale:.4f}",
              f"- hbm_bytes_per_launch: {hbm}",
              f"- kernel_source_sha256_16: `{src}`", ""]
    with open(COUNTERS_MD, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"hbm_bytes_per_launch": hbm, "fetch_scale": f_scale, "write_scale": w_scale}))
    return 0


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
    res = {
        "metric": "whole-model prefill input tokens/sec through streamed layer slots (1 MI355X, "
                  "host-link bound)",
        "value": wl.T / elapsed, "unit": "tokens/s", "n_gpus": 1, "steps": L, "warmup": 2,
        "ms_per_step": elapsed * 1e3 / L, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 x fp8_e4m3 (fp32 accumulate)" if a16 else "fp8_e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "slots": 2, "slot_bytes": slot_bytes,
                   "host_memory": "page-locked, one layer staged L times"},
        "h2d_GBs": L * slot_bytes / elapsed / 1e9,
        "per_layer_tokens_s": wl.T * L / elapsed,
    }
    print(json.dumps(res), flush=True)
    return 0


def cpu_baseline(layer, wl, x, ids, w, n_tokens, repeats, a16=False):
    """The oracle, as it stands, on the first n_tokens rows of the same batch:
    median wall clock of `repeats` runs."""
    import oracle
    import numpy as np
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
    return dict(value=n_tokens / dt, unit="tokens/s", cores=oracle.max_threads(), kind="oracle",
                sample=f"first {n_tokens} of the {wl.T} rows of the timed batch with all their "
                       f"routed experts{' (W8A16 form)' if a16 else ''}; median of {repeats} runs, "
                       f"{dt:.2f} s each")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="glm_e256_k8_h6144_i2048_t256")
    ap.add_argument("--cpu-tokens", type=int, default=256,
                    help="rows of the batch the CPU oracle is timed on (0 skips it)")
    ap.add_argument("--no-timing-events", action="store_true",
                    help="skip the per-launch HIP events (roofline needs them)")
    ap.add_argument("--cpu-repeats", type=int, default=3)
    ap.add_argument("--streamed-layers", type=int, default=0, metavar="L",
                    help="instead of the resident-layer bench: whole-model prefill through L layers "
                         "whose weights are staged from pinned host memory into two device slots "
                         "(double-buffered H2D overlapped with compute)")
    ap.add_argument("--decode", type=int, default=0, metavar="T",
                    help="time the W8A16 decode path (run_decode) on the first T rows of the "
                         "workload's batch instead of the W8A8 prefill path")
    ap.add_argument("--router", action="store_true",
                    help="start each step from FP32 router logits (run_logits: on-device top-k "
                         "router, then the path) instead of given ids and weights")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries from rocprofv3 CSV output under DIR")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.summarize_profiles:
        return summarize_profiles(args.summarize_profiles)
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
    if args.gpus != 1:
        print(json.dumps({"error": "this path runs on one GPU; multi-GPU sharding is design only "
                                   "(expert-parallel all-to-all), so --gpus must be 1"}))
        return 2

    import numpy as np
    import torch

    import fp8_blockwise_routed_amd as pkg
    import gen

    wl = gen.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    log(f"[bench] generating {wl.name}")
    t0 = time.perf_counter()
    layer = gen.make_layer(wl.E + wl.shared, wl.H, wl.I, seed=wl.seed)
    x, ids, w, _ = gen.make_inputs(wl)
    a16 = args.decode > 0
    if a16:  # the first T rows of the batch through the W8A16 decode path
        import dataclasses
        Td = min(args.decode, wl.T)
        x, ids, w = x[:Td], ids[:Td], w[:Td]
        wl = dataclasses.replace(wl, T=Td, name=f"{wl.name}_decode_t{Td}")
    log(f"[bench] generated in {time.perf_counter() - t0:.1f} s; creating the handle")
    moe = pkg.MoeFp8Prefill(layer, wl.k, routed_scale=wl.rho, max_rows=8192,
                            out_dtype=pkg.MOE_DTYPE_BF16, shared_experts=wl.shared)
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    idd = torch.from_numpy(ids).cuda()
    wd = torch.from_numpy(w).cuda()
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    if args.streamed_layers > 0:
        moe.close()
        return streamed_bench(args, wl, layer, xd, idd, wd, out)
    router = pkg.MOE_ROUTER_SOFTMAX if wl.route == gen.ROUTE_SOFTMAX else pkg.MOE_ROUTER_SIGMOID
    if args.router:
        logits = gen.make_logits(wl.T, wl.E, wl.route, wl.seed, wl.n_masked)
        ld = torch.from_numpy(logits).cuda()

    def step():
        if args.router:
            rc = pkg.moe_fp8_prefill_run_logits(moe.handle, xd, ld, router, wl.T, out, stream)
        elif a16:
            rc = pkg.moe_fp8_prefill_run_decode(moe.handle, xd, idd, wd, wl.T, out, stream)
        else:
            rc = pkg.moe_fp8_prefill_run(moe.handle, xd, idd, wd, wl.T, out, stream)
        if rc != pkg.MOE_OK:
            raise pkg.MoeError(rc, "run")

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    counts, _, _, _ = pkg.moe_fp8_prefill_debug_plan(moe.handle, wl.E + wl.shared,
                                                     wl.T * (wl.k + wl.shared))
    work = algorithmic_work(wl, counts, a16=a16)

    # Stage breakdown from a few untimed steps with events at every launch
    # boundary; they also name the dominant gate_up launch.
    timing = not args.no_timing_events
    stages, kind = None, None
    if timing:
        pkg.moe_fp8_prefill_set_timing(moe.handle, True)
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        stages = pkg.moe_fp8_prefill_read_timing(moe.handle)
        mean = stages.mean(axis=0)
        kind = max(("stream", "narrow", "wide"), key=lambda k: float(mean[pkg.STAGES.index("gate_up_" + k)]))
        if a16:
            kind = "decode"  # the W8A16 gate_up is timed in the streaming slot
        # in the timed steps, events only around that launch (two per step)
        pkg.moe_fp8_prefill_set_timing_stages(moe.handle, [gate_up_stage(kind)])
    log(f"[bench] timing {args.steps} steps")
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
    digest = hashlib.sha256(out.view(torch.int16).cpu().numpy().tobytes()).hexdigest()[:16]

    ms = elapsed * 1e3 / args.steps
    value = wl.T * args.steps / elapsed
    res = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": wl.name, "experts": wl.E, "top_k": wl.k, "hidden": wl.H,
                   "intermediate": wl.I, "rows": wl.T, "routed_scale": wl.rho,
                   "outlier_rows": wl.outlier_frac, "seed": wl.seed,
                   "shared_experts": wl.shared, "path": "decode (W8A16)" if a16 else "prefill (W8A8)"},
    }
    res["path"] = {
        "algorithmic_bytes": work["path_bytes"], "algorithmic_flops": work["path_flops"],
        "hbm_GBs": work["path_bytes"] / (ms * 1e-3) / 1e9,
        "hbm_frac": work["path_bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "mfma_TFLOPs": work["path_flops"] / (ms * 1e-3) / 1e12,
        "mfma_frac": work["path_flops"] / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
        "experts_hit": work["experts_hit"], "output_sha256_16": digest,
    }
    if stages is not None and len(stages) and live is not None and len(live):
        mean = stages.mean(axis=0)
        res["stages_ms"] = {name: float(v) for name, v in zip(pkg.STAGES, mean)}
        # the dominant gate_up launch, against the roof its algorithmic work
        # reaches first; its time from the events of the timed steps
        g = work["gate_up"][kind]
        launch_ms = float(live[:, pkg.STAGES.index(gate_up_stage(kind))].mean())
        mfma_peak = PEAK_BF16_TFLOPS if a16 else PEAK_FP8_TFLOPS
        t_hbm = g["bytes"] / (PEAK_HBM_GBS * 1e9)
        t_mfma = g["flops"] / (mfma_peak * 1e12)
        if t_mfma >= t_hbm:
            achieved = g["flops"] / (launch_ms * 1e-3) / 1e12
            bound, peak, unit = "mfma", mfma_peak, "TFLOP/s"
        else:
            achieved = g["bytes"] / (launch_ms * 1e-3) / 1e9
            bound, peak, unit = "hbm", PEAK_HBM_GBS, "GB/s"
        res["roofline"] = {
            "kernel": GATE_UP_KERNELS[kind],
            "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "traffic": read_traffic() if kind == "stream" else None,
            "algorithmic_bytes_per_launch": g["bytes"],
            "algorithmic_flops_per_launch": g["flops"],
            "experts_in_launch": g["experts"], "rows_in_launch": g["rows"],
            "avg_launch_ms": launch_ms,
        }
    if args.router:
        # the router alone, timed with HIP events on the run stream
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
                         "avg_launch_us": r_us, "algorithmic_bytes": r_bytes,
                         "GBs": r_bytes / (r_us * 1e-6) / 1e9,
                         "ids_equal_given": bool(torch.equal(ids_r, idd))}
        res["config"]["input"] = "router logits"
    if args.cpu_tokens > 0:
        log(f"[bench] CPU oracle on {args.cpu_tokens} rows")
        res["cpu_baseline"] = cpu_baseline(layer, wl, x, ids, w, min(args.cpu_tokens, wl.T),
                                           a16=a16, repeats=max(1, args.cpu_repeats))
    moe.close()
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
