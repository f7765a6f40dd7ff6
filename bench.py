#!/usr/bin/env python3
"""Benchmark of the fused QK-RMSNorm + RoPE (+ V) prologue on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one launch of the whole prologue (norm, rotation, V copy, output rounding) over one
batch of the workload. The default workload is the 15360-token, 32-head, head_dim-128 3D problem
with across-heads norm and interleaved pairs (LTX-2's video self-attention shape). Inputs are
seeded synthetic bf16 drawn by qk_rmsnorm_rope_amd.workloads, resident in HBM before timing.
Prints one JSON line with tokens/s, the HBM roofline of the kernel and a CPU baseline (the fp64
oracle on a bounded sample of the same workload).

Other modes (used to produce the committed profiles):
    --profile-run       only warmup + steps launches, no CPU baseline, no JSON line
    --copy-calibration  launches a plain elementwise copy of known size (counter calibration)
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

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak, GB/s
DEFAULT_WORKLOAD = "rope3d_across_interleaved_s15360_h32_d128"
KERNEL_SOURCES = ["qk_rmsnorm_rope_amd/csrc/qkrope_kernel_impl.h",
                  "qk_rmsnorm_rope_amd/csrc/qkrope_internal.h",
                  "qk_rmsnorm_rope_amd/csrc/qkrope_api.cpp"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w) -> int:
    """Bytes the method itself must move per launch: inputs read once, outputs written once."""
    if hasattr(w, "row_elems"):             # 3D form
        T = w.num_tokens
        out_b = 1 if w.output_fp8 else 2
        read = T * w.row_elems * 2
        if w.is_qk_norm:
            read += (w.num_heads_q + w.num_heads_k) * w.head_dim * 2
        return read + T * w.row_elems * out_b
    T, D = w.num_tokens, w.head_dim
    qk = T * (w.num_heads_q + w.num_heads_k) * D * 2
    tab = T * w.rotary_dim * (4 if w.table_dtype == "f32" else 2)
    wts = 0 if w.norm_mode == "none" else 2 * D * 2
    return qk + tab + wts + qk


def traffic_from_profile(w) -> dict | None:
    """Counter-measured HBM bytes per launch from profiles/counters_<workload>.md, if taken on
    the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"counters_{w.name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"<!--\s*traffic\s+(\{.*?\})\s*-->", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec


def make_launcher(w, dev, sets):
    """Inputs/outputs on the GPU (`sets` copies, rotated per launch) and a launch closure.

    Launch arguments are marshalled once per buffer set (qk_rmsnorm_rope_amd.Prepared3D and
    PreparedTable), so the timed loop is one C call per step and the GPU queue never runs dry
    on host overhead."""
    import torch
    import qk_rmsnorm_rope_amd as qr
    from qk_rmsnorm_rope_amd import workloads as wl

    calls = []
    if hasattr(w, "row_elems"):
        cpu = wl.rope3d_inputs(w)
        for _ in range(sets):
            g = {k: v.to(dev) for k, v in cpu.items()}
            outs = qr.run_workload_3d(w, g["qkv"], g["q_weight"], g["k_weight"])
            calls.append(qr.Prepared3D(w, g["qkv"], g["q_weight"], g["k_weight"], *outs))
    else:
        cpu = wl.table_inputs(w)
        for _ in range(sets):
            g = {k: v.to(dev) for k, v in cpu.items()}
            qo, ko = torch.empty_like(g["q"]), torch.empty_like(g["k"])
            calls.append(qr.PreparedTable(g["q"], g["k"], g["q_weight"], g["k_weight"],
                                          g["rope_table"], w.eps, q_out=qo, k_out=ko,
                                          rotary_dim=w.rotary_dim, interleaved=w.interleaved,
                                          norm_mode=w.norm_mode))

    def launch(i):
        calls[i % sets]()
    return cpu, launch


def time_launches(launch, steps, warmup):
    """Warm up, then time `steps` back-to-back launches: wall clock between two synchronisations,
    and HIP events recorded on the launch stream around the whole timed region. Returns
    (wall_s, gpu_s_per_launch)."""
    import torch
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        launch(warmup + i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) * 1e-3 / steps


def cpu_baseline(w, cpu_inputs, budget_s: float = 12.0) -> dict:
    """The fp64 oracle, as it stands, on the first tokens of the same workload (output encoding
    included), on every host core OpenMP gives it, until `budget_s` of work."""
    import numpy as np
    import oracle

    threads = oracle.num_threads()
    done, t_used, chunk = 0, 0.0, 64
    if hasattr(w, "row_elems"):
        x = cpu_inputs["qkv"].reshape(-1, w.row_elems)
        limit = w.num_tokens
    else:
        limit = w.num_tokens
    while t_used < budget_s and done < limit:
        n = min(chunk, limit - done)
        t0 = time.perf_counter()
        if hasattr(w, "row_elems"):
            q, k, v = oracle.run_3d_workload(w, x[done:done + n], cpu_inputs["q_weight"],
                                             cpu_inputs["k_weight"], token_offset=done)
            if w.output_fp8:
                oracle.e4m3_encode(q, w.output_quant_scale)
                oracle.e4m3_encode(k, w.output_quant_scale)
                oracle.e4m3_encode(v, w.v_quant_scale)
            else:
                oracle.bf16_encode(q), oracle.bf16_encode(k), oracle.bf16_encode(v)
        else:
            q, k = oracle.run_table(cpu_inputs["q"][done:done + n], cpu_inputs["k"][done:done + n],
                                    cpu_inputs["q_weight"], cpu_inputs["k_weight"],
                                    cpu_inputs["rope_table"][done:done + n], w.eps,
                                    rotary_dim=w.rotary_dim, interleaved=w.interleaved,
                                    norm_mode=w.norm_mode)
            oracle.bf16_encode(q), oracle.bf16_encode(k)
        t_used += time.perf_counter() - t0
        done += n
        chunk = min(chunk * 2, 4096)
    return {"value": done / t_used, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {done} of {limit} tokens of {w.name}, fp64 oracle incl. output "
                      f"encoding, {t_used:.1f} s on {threads} OpenMP threads",
            "gbs": algorithmic_bytes(w) * done / limit / t_used / 1e9}


def copy_calibration(dev, steps, warmup):
    """A plain elementwise copy of a known size (1 GiB read + 1 GiB written per launch)."""
    import torch
    n = 1 << 29
    x = torch.randn(n, device=dev).to(torch.bfloat16)
    y = torch.empty_like(x)
    total, mean = time_launches(lambda i: torch.neg(x, out=y), steps, warmup)
    print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n,
                      "mean_launch_us": mean * 1e6, "gbs": 4 * n / mean / 1e9}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--sets", type=int, default=3,
                    help="input/output buffer sets rotated across launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the prologue is token-local and this build runs on a "
              "single MI355X (no multi-GPU path); use --gpus 1", file=sys.stderr)
        return 2

    import torch
    from qk_rmsnorm_rope_amd import workloads as wl

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(dev, args.steps, args.warmup)
        return 0
    w = wl.WORKLOADS[args.workload]
    cpu_inputs, launch = make_launcher(w, dev, args.sets)
    torch.cuda.synchronize()
    total, mean_launch = time_launches(launch, args.steps, args.warmup)
    if args.profile_run:
        print(f"{w.name}: {args.steps} launches, mean {mean_launch * 1e6:.1f} us", flush=True)
        return 0

    nbytes = algorithmic_bytes(w)
    ms_per_step = total / args.steps * 1e3
    achieved = nbytes / mean_launch / 1e9
    traffic = traffic_from_profile(w)
    result = {
        "metric": "tokens/s and achieved HBM GB/s (% of peak) for fused QK-RMSNorm+RoPE+V",
        "value": w.num_tokens / (total / args.steps),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.num_tokens, "io_dtype": "bf16",
                   "heads": [w.num_heads_q, w.num_heads_k, getattr(w, "num_heads_v", 0)],
                   "head_dim": w.head_dim, "parallelism": "single-gpu",
                   "buffer_sets": args.sets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic["bytes_per_launch"] if traffic else None,
                     "algorithmic_bytes": nbytes, "mean_launch_us": mean_launch * 1e6},
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, cpu_inputs)
        result["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
