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
METRIC = "input tokens/sec per MoE layer (1 MI355X) + % FP8 MFMA peak / % HBM peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_small_glm_t256_traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "fp8_blockwise_routed_amd", "csrc", "moe_kernels.hip")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def algorithmic_work(wl, counts):
    """Algorithmic bytes / FLOPs from the plan's per-expert row counts.

    Per expert with n_e > 0 rows: weights 3*Ip*H code bytes + FP32 block
    scales 4*(2*nI*nH + nH*nI); per routed slot: 6*Ip*H FLOPs.  Plus the
    input rows (T*H*2) and output rows (T*H*2 for BF16) and ids/weights (8*P).
    Returns the whole path and the gate_up 1-subtile launch (experts with
    1..16 rows): its weights 2*Ip*H + 8*nI*nH per expert, the activation row
    (H + 4*nH) read and the h row (Ip + 4*nI) written per slot.
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
    small = (counts >= 1) & (counts <= 16)
    n_small = int(counts[small].sum())
    gu_bytes = int(small.sum()) * (2 * Ip * H + 8 * nI * nH) + n_small * (H + 4 * nH + Ip + 4 * nI)
    gu_flops = 4 * n_small * Ip * H
    return dict(path_bytes=path_bytes, path_flops=path_flops, gu_small_bytes=gu_bytes,
                gu_small_flops=gu_flops, experts_hit=int(hit.sum()), experts_small=int(small.sum()),
                slots=P, per_expert_gate_up_bytes=2 * Ip * H + 8 * nI * nH)


def read_traffic(n_launch_bytes):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, or None if absent or taken on different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(layer, wl, x, ids, w, n_tokens):
    """The oracle, as it stands, on the first n_tokens rows of the same batch."""
    import oracle
    t0 = time.perf_counter()
    oracle.forward(layer, x[:n_tokens], ids[:n_tokens], w[:n_tokens], wl.rho, oracle.OUT_BF16)
    dt = time.perf_counter() - t0
    return dict(value=n_tokens / dt, unit="tokens/s", cores=oracle.max_threads(), kind="oracle",
                sample=f"first {n_tokens} of the {wl.T} rows of the timed batch "
                       f"(all their routed experts), wall clock {dt:.2f} s")


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
    args = ap.parse_args()
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
    layer = gen.make_layer(wl.E, wl.H, wl.I, seed=wl.seed)
    x, ids, w, _ = gen.make_inputs(wl)
    log(f"[bench] generated in {time.perf_counter() - t0:.1f} s; creating the handle")
    moe = pkg.MoeFp8Prefill(layer, wl.k, routed_scale=wl.rho, max_rows=8192,
                            out_dtype=pkg.MOE_DTYPE_BF16)
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    idd = torch.from_numpy(ids).cuda()
    wd = torch.from_numpy(w).cuda()
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        rc = pkg.moe_fp8_prefill_run(moe.handle, xd, idd, wd, wl.T, out, stream)
        if rc != pkg.MOE_OK:
            raise pkg.MoeError(rc, "run")

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    counts, _, _, _ = pkg.moe_fp8_prefill_debug_plan(moe.handle, wl.E, wl.T * wl.k)
    work = algorithmic_work(wl, counts)

    timing = not args.no_timing_events
    pkg.moe_fp8_prefill_set_timing(moe.handle, timing)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stages = pkg.moe_fp8_prefill_read_timing(moe.handle) if timing else None
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
                   "outlier_rows": wl.outlier_frac, "seed": wl.seed},
    }
    res["path"] = {
        "algorithmic_bytes": work["path_bytes"], "algorithmic_flops": work["path_flops"],
        "hbm_GBs": work["path_bytes"] / (ms * 1e-3) / 1e9,
        "hbm_frac": work["path_bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "mfma_TFLOPs": work["path_flops"] / (ms * 1e-3) / 1e12,
        "mfma_frac": work["path_flops"] / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
        "experts_hit": work["experts_hit"], "output_sha256_16": digest,
    }
    if stages is not None and len(stages):
        mean = stages.mean(axis=0)
        res["stages_ms"] = {name: float(v) for name, v in zip(pkg.STAGES, mean)}
        gu_ms = float(mean[pkg.STAGES.index("gate_up_small")])
        achieved = work["gu_small_bytes"] / (gu_ms * 1e-3) / 1e9
        traffic = read_traffic(work["gu_small_bytes"])
        res["roofline"] = {
            "kernel": "gate_up_kernel<1> (experts with 1..16 rows)",
            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
            "algorithmic_bytes_per_launch": work["gu_small_bytes"],
            "experts_in_launch": work["experts_small"],
            "avg_launch_ms": gu_ms,
        }
    if args.cpu_tokens > 0:
        log(f"[bench] CPU oracle on {args.cpu_tokens} rows")
        res["cpu_baseline"] = cpu_baseline(layer, wl, x, ids, w, min(args.cpu_tokens, wl.T))
    moe.close()
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
