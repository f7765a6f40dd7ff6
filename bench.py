#!/usr/bin/env python3
"""Benchmark of the fused QK-RMSNorm + RoPE (+ V) prologue on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one launch of the whole prologue (norm, rotation, V copy, output rounding) over one
batch of the workload. The timed steps are captured once into a HIP graph and replayed (the way
a fixed-shape prologue that runs in every layer and denoising step is launched in production);
--stream launches them one by one from the host instead.
The default workload is the largest one that fits one GPU: 122880 tokens of packed bf16 QKV,
16 heads of 256 each, 3D RoPE with YaRN and no norm (6.04 GB moved per step). In the same run,
and in the same JSON line under "also_timed", the two other workloads held to the bandwidth
target are timed the same way: the 15360-token, 32-head, head_dim-128 3D problem with
across-heads norm (LTX-2's video self-attention shape) and the 2 x 18480-token, 20-head,
head_dim-64 NeoX problem with E4M3 outputs (SANA-WM's grid). Inputs are seeded synthetic bf16
drawn by qk_rmsnorm_rope_amd.workloads, resident in HBM before timing.
Prints one JSON line with tokens/s, the HBM roofline of the kernel and a CPU baseline (the fp64
oracle on a bounded sample of the headline workload).

Other modes (used to produce the committed profiles):
    --profile-run       only warmup + steps launches, no CPU baseline, no JSON line
    --copy-calibration  launches a plain elementwise copy of known size (counter calibration)
    --crossover         fused table-form call vs an eager torch chain over 64..65536 tokens (the
                        fused-vs-eager threshold of vLLM-Omni's fused_qk_norm_rope_min_tokens)
    --stream            launch each step on the stream from the host instead of replaying the
                        timed steps as one HIP graph (the default)
    --cold              rotate enough input/output buffer sets that they total at least 512 MB
                        (twice the 256 MB memory-side cache), so no launch finds its data cached;
                        the default three sets already exceed that for the large workloads
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
COLD_BYTES = 512 << 20         # --cold: rotating buffer sets total at least twice the MALL
DEFAULT_WORKLOAD = "rope3d_yarn_nonorm_s122880_h16_d256"
# timed after the default workload, in the same run, as sub-records of its JSON line
ALSO_TIMED = ("rope3d_across_interleaved_s15360_h32_d128", "rope3d_neox_fp8_b2_s18480_h20_d64")
_CSRC = "qk_rmsnorm_rope_amd/csrc/"
# build.py holds the compile flags; the per-variant .hip files choose the instantiations
COMMON_SOURCES = [_CSRC + "qkrope_kernel_impl.h", _CSRC + "qkrope_internal.h",
                  _CSRC + "qkrope_host.h", "qk_rmsnorm_rope_amd/build.py"]
PROLOGUE_SOURCES = [_CSRC + "qkrope_api.cpp"] + sorted(
    _CSRC + f for f in os.listdir(os.path.join(ROOT, _CSRC))
    if f.startswith("qkrope_kernels_") and f.endswith(".hip") and "cam" not in f)
CAM_SOURCES = [_CSRC + "qkrope_cam.h", _CSRC + "qkrope_api_cam.cpp",
               _CSRC + "qkrope_kernels_cam.hip"]


_COMMENTS = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)
_PY_COMMENTS = re.compile(r"#[^\n]*")


def kernel_source_hash(w=None) -> str:
    """Hash of the code of the sources that decide a workload's kernel and launch shape, with
    comments and whitespace dropped (a record survives an edit of comments only)."""
    h = hashlib.sha256()
    cam = w is not None and is_cam(w)
    for rel in COMMON_SOURCES + (CAM_SOURCES if cam else PROLOGUE_SOURCES):
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = (_PY_COMMENTS if rel.endswith(".py") else _COMMENTS).sub(" ", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def is_3d(w) -> bool:
    return hasattr(w, "row_elems")


def is_cam(w) -> bool:
    return hasattr(w, "k_scale")


def total_tokens(w) -> int:
    """Tokens one step processes (the camera prologue's batch counts its tokens once each)."""
    return w.batch * w.num_tokens if is_cam(w) else w.num_tokens


def kernel_name(w) -> str:
    """Name fragment of the step's dominant kernel in profiler output."""
    return "qkrope_cam_kernel" if is_cam(w) else "qkrope_kernel"


def is_sharded(w) -> bool:
    return is_3d(w) and w.head_shards > 1


def algorithmic_bytes(w) -> int:
    """Bytes the method itself must move per launch of the step's dominant kernel: inputs read
    once, outputs written once (for a head-sharded rank: the apply kernel, which also reads the
    [T, 2] fp32 sums; for the camera prologue: Q, K, V in and out, the per-token 4x4 fp32
    matrices, the [N, D/2] fp32 cos and sin tables once, inflation_sq out)."""
    if is_cam(w):
        BN, H, D = w.batch * w.num_tokens, w.num_heads, w.head_dim
        return BN * (12 * H * D + 4 * H + 2 * 64) + w.num_tokens * 4 * D
    if is_3d(w):
        T = w.num_tokens
        out_b = 1 if w.output_fp8 else 2
        read = T * w.row_elems * 2
        if w.is_qk_norm:
            read += (w.num_heads_q + w.num_heads_k) * w.head_dim * 2
            if is_sharded(w):
                read += T * 8
        return read + T * w.row_elems * out_b
    T, D = w.num_tokens, w.head_dim
    qk = T * (w.num_heads_q + w.num_heads_k) * D * 2
    tab = T * w.rotary_dim * (4 if w.table_dtype == "f32" else 2)
    wts = {"none": 0, "per_head": 2 * D * 2,
           "across_heads": (w.num_heads_q + w.num_heads_k) * D * 2}[w.norm_mode]
    out = qk // 2 if w.out_dtype == "e4m3" else qk
    return qk + tab + wts + out


def output_bytes(w) -> int:
    """The part of algorithmic_bytes(w) that is written."""
    if is_cam(w):
        BN, H, D = w.batch * w.num_tokens, w.num_heads, w.head_dim
        return BN * (6 * H * D + 4 * H)
    if is_3d(w):
        return w.num_tokens * w.row_elems * (1 if w.output_fp8 else 2)
    return w.num_tokens * (w.num_heads_q + w.num_heads_k) * w.head_dim * \
        (1 if w.out_dtype == "e4m3" else 2)


def sumsq_bytes(w) -> int:
    """Algorithmic bytes of the per-token sum-of-squares kernel of a head-sharded rank."""
    return w.num_tokens * ((w.num_heads_q + w.num_heads_k) * w.head_dim * 2 + 8)


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
    if rec.get("kernel_source_hash") != kernel_source_hash(w):
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
    if is_cam(w):
        cpu = wl.cam_inputs(w)
        B, N, H, D = w.batch, w.num_tokens, w.num_heads, w.head_dim
        for _ in range(sets):
            g = {k: v.to(dev) for k, v in cpu.items()}
            outs = [torch.empty((B, H, D, N), dtype=g["q"].dtype, device=dev) for _ in range(3)]
            infl = torch.empty((B, H, N), dtype=torch.float32, device=dev)
            calls.append(qr.PreparedCam(g["q"], g["k"], g["v"], g["proj_q"], g["proj_kv"],
                                        g["rope_cos"], g["rope_sin"], w.k_scale, *outs, infl))
    elif is_sharded(w):
        # one rank: the all-reduce of the sums over the head group is the identity, so the
        # apply kernel reads the rank's own sums (same bytes and arithmetic as the reduced ones)
        cpu = wl.rope3d_inputs(w)
        for _ in range(sets):
            g = {k: v.to(dev) for k, v in cpu.items()}
            odt = torch.float8_e4m3fn if w.output_fp8 else torch.bfloat16
            outs = [torch.empty((w.num_tokens, H, w.head_dim), dtype=odt, device=dev)
                    for H in (w.num_heads_q, w.num_heads_k, w.num_heads_v)]
            ss = torch.empty((w.num_tokens, 2), dtype=torch.float32, device=dev)
            calls.append(qr.PreparedSharded3D(w, g["qkv"], g["q_weight"], g["k_weight"], *outs,
                                              ss, ss))
    elif is_3d(w):
        cpu = wl.rope3d_inputs(w)
        for _ in range(sets):
            g = {k: v.to(dev) for k, v in cpu.items()}
            outs = qr.run_workload_3d(w, g["qkv"], g["q_weight"], g["k_weight"])
            calls.append(qr.Prepared3D(w, g["qkv"], g["q_weight"], g["k_weight"], *outs))
    else:
        cpu = wl.table_inputs(w)
        for _ in range(sets):
            g = {k: v.to(dev) for k, v in cpu.items()}
            odt = torch.float8_e4m3fn if w.out_dtype == "e4m3" else g["q"].dtype
            qo = torch.empty(g["q"].shape, dtype=odt, device=dev)
            ko = torch.empty(g["k"].shape, dtype=odt, device=dev)
            calls.append(qr.PreparedTable(g["q"], g["k"], g["q_weight"], g["k_weight"],
                                          g["rope_table"], w.eps, q_out=qo, k_out=ko,
                                          rotary_dim=w.rotary_dim, interleaved=w.interleaved,
                                          norm_mode=w.norm_mode, out_scale=w.out_scale))

    def launch(i):
        calls[i % sets]()
    return cpu, launch, calls


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


def time_graph(launch, steps, warmup):
    """Capture `steps` launches in one HIP graph on the current stream and time one replay:
    (wall_s, gpu_s_per_launch), like time_launches."""
    import torch
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.current_stream()):
        for i in range(steps):
            launch(warmup + i)
    graph.replay()                                  # warm replay
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    graph.replay()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) * 1e-3 / steps


def host_cpu() -> str:
    """The host CPU's model name (Linux), or "unknown CPU"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(w, cpu_inputs, budget_s: float = 12.0) -> dict:
    """The fp64 oracle, as it stands, on the same workload's tokens in order (output encoding
    included, starting again from the first token after the last), on every host core OpenMP
    gives it, until `budget_s` of work."""
    import oracle

    threads = oracle.num_threads()
    done, t_used, chunk = 0, 0.0, 64
    if is_3d(w):
        x = cpu_inputs["qkv"].reshape(-1, w.row_elems)
    limit = w.num_tokens                # per batch for the camera prologue (all batches run)
    total = 0
    while t_used < budget_s:
        if done == limit:               # whole workload done: another pass
            done = 0
        n = min(chunk, limit - done)
        t0 = time.perf_counter()
        if is_cam(w):
            sl = slice(done, done + n)
            outs = oracle.cam_prep(*(cpu_inputs[k][:, sl].contiguous() for k in
                                     ("q", "k", "v", "proj_q", "proj_kv")),
                                   cpu_inputs["rope_cos"][sl].contiguous(),
                                   cpu_inputs["rope_sin"][sl].contiguous(), w.k_scale)
            enc = oracle.f16_encode if w.act_dtype == "f16" else oracle.bf16_encode
            enc(outs[0]), enc(outs[1]), enc(outs[2])
        elif is_3d(w):
            if is_sharded(w):
                oracle.sumsq_3d(x[done:done + n], num_heads_q=w.num_heads_q,
                                num_heads_k=w.num_heads_k, num_heads_v=w.num_heads_v,
                                head_dim=w.head_dim)
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
            if w.out_dtype == "e4m3":
                oracle.e4m3_encode(q, w.out_scale), oracle.e4m3_encode(k, w.out_scale)
            elif w.act_dtype == "f16":
                oracle.f16_encode(q), oracle.f16_encode(k)
            else:
                oracle.bf16_encode(q), oracle.bf16_encode(k)
        t_used += time.perf_counter() - t0
        done += n
        total += n
        chunk = min(chunk * 2, 4096)
    nb = w.batch if is_cam(w) else 1
    what = (f"{total} tokens ({total / limit:.2f} passes over the {limit} tokens"
            + (f" of each of {nb} batches" if is_cam(w) else "") + ")")
    return {"value": nb * total / t_used, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} of {w.name}, fp64 oracle incl. output "
                      f"encoding, {t_used:.1f} s on {threads} OpenMP threads "
                      f"({host_cpu()}, {os.cpu_count()} logical CPUs)",
            "gbs": algorithmic_bytes(w) * total / limit / t_used / 1e9}


def copy_calibration(dev, steps, warmup):
    """A plain elementwise copy of a known size (1 GiB read + 1 GiB written per launch)."""
    import torch
    n = 1 << 29
    x = torch.randn(n, device=dev).to(torch.bfloat16)
    y = torch.empty_like(x)
    total, mean = time_launches(lambda i: torch.neg(x, out=y), steps, warmup)
    print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n,
                      "mean_launch_us": mean * 1e6, "gbs": 4 * n / mean / 1e9}), flush=True)


def eager_table_chain(q, k, q_weight, k_weight, table, eps, rotary_dim, interleaved):
    """The unfused chain a consumer keeps below the fused-vs-eager threshold: torch's RMSNorm
    per head, then RoPE from the packed [cos | sin] table with torch elementwise ops, in fp32,
    rounded back to the activation dtype (several kernel launches per call). A timing
    comparator only; correctness is judged against the oracle elsewhere."""
    import torch
    import torch.nn.functional as F
    R, D = rotary_dim, q.shape[-1]
    cos = table[:, : R // 2].float().unsqueeze(1)
    sin = table[:, R // 2: R].float().unsqueeze(1)
    outs = []
    for x, w in ((q, q_weight), (k, k_weight)):
        n = F.rms_norm(x.float(), (D,), w.float(), eps)
        if interleaved:
            a, b = n[..., 0:R:2], n[..., 1:R:2]
            rot = torch.stack((a * cos - b * sin, b * cos + a * sin), dim=-1).flatten(-2)
        else:
            a, b = n[..., : R // 2], n[..., R // 2: R]
            rot = torch.cat((a * cos - b * sin, b * cos + a * sin), dim=-1)
        outs.append(torch.cat((rot, n[..., R:]), dim=-1).to(x.dtype))
    return tuple(outs)


def crossover(dev, warmup) -> None:
    """Per-call wall time of the fused table-form call (through the page's signature, outputs
    allocated per call as a consumer does), of the eager chain, and of the fused call marshalled
    once beforehand (PreparedTable: one C call, the floor of the host cost), for 64..65536 tokens
    of the 24-head, head_dim-128 interleaved workload with a bf16 table; one JSON line per size,
    then the smallest size from which on the fused call is never slower than the eager chain."""
    import torch
    import qk_rmsnorm_rope_amd as qr
    from qk_rmsnorm_rope_amd import workloads as wl

    sizes = [64 << i for i in range(11)]
    w = wl.TABLE_INTERLEAVED_T4096.with_(num_tokens=sizes[-1])
    g = {k: v.to(dev) for k, v in wl.table_inputs(w).items()}
    rows = []
    for T in sizes:
        q, k, tab = g["q"][:T], g["k"][:T], g["rope_table"][:T]
        args = (q, k, g["q_weight"], g["k_weight"], tab, w.eps)
        fused = lambda: qr.fused_qk_norm_rope(*args, rotary_dim=w.rotary_dim, interleaved=True)
        eager = lambda: eager_table_chain(*args, w.rotary_dim, True)
        # reference: the same call marshalled once, outputs allocated once (one C call)
        prepared = qr.PreparedTable(*args, q_out=torch.empty_like(q), k_out=torch.empty_like(k),
                                    rotary_dim=w.rotary_dim, interleaved=True)
        if T == sizes[0]:
            a, b = fused(), eager()
            torch.cuda.synchronize()
            assert all((x.float() - y.float()).abs().max().item() < 0.05 for x, y in zip(a, b))
        n = max(20, min(2000, (1 << 22) // T))
        res = {"tokens": T, "calls": n}
        for name, fn in (("fused_us", fused), ("eager_us", eager), ("prepared_us", prepared)):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
            res[name] = (time.perf_counter() - t0) / n * 1e6
        rows.append(res)
        print(json.dumps(res), flush=True)
    cross = None
    for i in range(len(rows)):
        if all(r["fused_us"] <= r["eager_us"] for r in rows[i:]):
            cross = rows[i]["tokens"]
            break
    print(json.dumps({"crossover_tokens": cross, "note": "smallest measured size from which "
                      "the fused call is never slower than the eager chain"}), flush=True)


def measure(w, dev, args, use_graph):
    """Prepare `args.sets` buffer sets of workload `w` on `dev` and time it as bench.py does.
    Returns (cpu_inputs, wall_s_total, s_per_step, s_per_launch of the dominant kernel, extra)."""
    import torch
    sets = args.sets
    if args.cold:
        sets = max(sets, -(-COLD_BYTES // algorithmic_bytes(w)))
    timer = time_graph if use_graph else time_launches
    cpu_inputs, launch, calls = make_launcher(w, dev, sets)
    torch.cuda.synchronize()
    total, mean_step = timer(launch, args.steps, args.warmup)
    mean_launch = mean_step
    extra = {"buffer_sets": sets}
    if is_sharded(w):
        # the step is two kernels: time each on its own for the per-kernel rooflines
        _, mean_launch = timer(lambda i: calls[i % sets].apply(), args.steps, args.warmup)
        _, mean_sumsq = timer(lambda i: calls[i % sets].sumsq(), args.steps, args.warmup)
        extra.update({"sumsq_kernel": {"achieved": sumsq_bytes(w) / mean_sumsq / 1e9,
                                       "unit": "GB/s", "mean_launch_us": mean_sumsq * 1e6,
                                       "algorithmic_bytes": sumsq_bytes(w)},
                      "apply_kernel_us": mean_launch * 1e6, "step_us": mean_step * 1e6})
    del launch, calls
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return cpu_inputs, total, mean_step, mean_launch, extra


def roofline(w, mean_launch) -> dict:
    nbytes = algorithmic_bytes(w)
    achieved = nbytes / mean_launch / 1e9
    traffic = traffic_from_profile(w)
    return {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic["bytes_per_launch"] if traffic else None,
            "algorithmic_bytes": nbytes, "mean_launch_us": mean_launch * 1e6}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--sets", type=int, default=3,
                    help="input/output buffer sets rotated across launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true",
                    help="time only the default workload (skip the also_timed sub-records)")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--crossover", action="store_true")
    ap.add_argument("--stream", action="store_true")
    ap.add_argument("--cold", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the prologue is token-local and the library runs on "
              "a single MI355X (no multi-GPU path); use --gpus 1", file=sys.stderr)
        return 2

    import torch
    from qk_rmsnorm_rope_amd import workloads as wl

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(dev, args.steps, args.warmup)
        return 0
    if args.crossover:
        crossover(dev, args.warmup)
        return 0
    w = wl.WORKLOADS[args.workload]
    use_graph = not args.stream
    if use_graph:
        # launchers bind the stream they are prepared on: prepare them on the capture stream
        capture = torch.cuda.Stream()
        capture.wait_stream(torch.cuda.current_stream())
        torch.cuda.set_stream(capture)
    cpu_inputs, total, mean_step, mean_launch, extra = measure(w, dev, args, use_graph)
    sets = extra.pop("buffer_sets")
    if args.profile_run:
        print(f"{w.name}: {args.steps} launches, mean {mean_step * 1e6:.1f} us", flush=True)
        return 0

    also = []
    if args.workload == DEFAULT_WORKLOAD and not args.no_also:
        for name in ALSO_TIMED:
            wa = wl.WORKLOADS[name]
            _, t_a, step_a, launch_a, ex_a = measure(wa, dev, args, use_graph)
            also.append({"workload": name, "tokens": total_tokens(wa),
                         "value": total_tokens(wa) / (t_a / args.steps), "unit": "tokens/s",
                         "ms_per_step": t_a / args.steps * 1e3,
                         "buffer_sets": ex_a["buffer_sets"], "roofline": roofline(wa, launch_a)})

    ms_per_step = total / args.steps * 1e3
    result = {
        "metric": "tokens/s and achieved HBM GB/s (% of peak) for fused QK-RMSNorm+RoPE+V",
        "value": total_tokens(w) / (total / args.steps),
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
        "config": {"workload": w.name, "tokens": total_tokens(w),
                   "io_dtype": getattr(w, "act_dtype", "bf16"),
                   "heads": ([w.num_heads] * 3 if is_cam(w) else
                             [w.num_heads_q, w.num_heads_k, getattr(w, "num_heads_v", 0)]),
                   "head_dim": w.head_dim,
                   "parallelism": (f"one rank of {w.head_shards} head shards"
                                   if is_sharded(w) else "single-gpu"),
                   "buffer_sets": sets,
                   "launch": "hip_graph" if use_graph else "stream"},
        "roofline": roofline(w, mean_launch),
        **extra,
    }
    if also:
        result["also_timed"] = also
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, cpu_inputs)
        result["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
