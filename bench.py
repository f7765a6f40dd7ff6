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
head_dim-64 NeoX problem with E4M3 outputs (SANA-WM's grid); so is the SANA-WM camera prologue
on that grid (2 x 18480 tokens, 20 heads of 64, outputs transposed to [B, H, D, N]). Inputs are
seeded synthetic bf16
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
# timed after the default workload, in the same run, as sub-records of its JSON line: the two
# other 3D workloads held to the bandwidth target, and the SANA-WM camera prologue
ALSO_TIMED = ("rope3d_across_interleaved_s15360_h32_d128", "rope3d_neox_fp8_b2_s18480_h20_d64",
              "cam_prep_b2_s18480_h20_d64")
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
            # rows of w.out_pitch elements, of which the op writes the first N
            outs = [torch.empty((B, H, D, w.out_pitch), dtype=g["q"].dtype, device=dev)[..., :N]
                    for _ in range(3)]
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


# --- profiles: rocprofv3 passes over bench.py's own sequences, and their summaries -------------
#
# `bench.py --profile-workload NAME [--profile-dir DIR]` runs, each as a child process under
# rocprofv3 (from /tmp, TMPDIR=/tmp), a kernel trace of bench.py's timed sequence and four
# counter passes of a short stream-launched sequence, then writes profiles/counters_NAME.md
# (kernel durations, HBM bytes per dispatch against the algorithmic bytes, and the traffic
# record bench.py reports) and profiles/sq_NAME.md (instruction mix, VALU busy, LDS bank
# conflicts). `--profile-workload copy` profiles the plain copy that calibrates the byte
# counters (profiles/copy_calibration.md); it is read by every other summary, so profile it
# first. Raw rocprofv3 output stays in DIR.

PMC_PASSES = {
    "fetch": ["FETCH_SIZE"],
    # WRITE_SIZE is built from these two: 64-byte and 32-byte write requests
    "write": ["WRITE_SIZE", "TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum"],
    # read requests by size: FETCH_SIZE's expression weighs each 128-byte request as 64 bytes
    # unless TCC_BUBBLE counts it, so its calibration is cross-checked from the request sizes
    "rdreq": ["TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum",
              "TCC_EA0_RDREQ_128B_sum"],
    "sq": ["SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_WAVES", "SQ_ACTIVE_INST_VALU",
           "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"],
}
COPY_KERNEL = "vectorized_elementwise_kernel<8"   # torch's copy in --copy-calibration
COPY_TRACE_STEPS = 20                              # timed copies in its kernel trace


def _rel(path: str) -> str:
    return os.path.relpath(path, ROOT)


def profile_commands(name: str, out_dir: str) -> dict:
    """The rocprofv3 command of each pass (argv lists, paths absolute)."""
    bench = os.path.join(ROOT, "bench.py")
    if name == "copy":
        prog = ["python3", bench, "--copy-calibration", "--steps", str(COPY_TRACE_STEPS),
                "--warmup", "5"]
        prog_pmc = ["python3", bench, "--copy-calibration", "--steps", "5", "--warmup", "2"]
    else:
        prog = ["python3", bench, "--workload", name, "--profile-run", "--steps", "100",
                "--warmup", "20"]
        prog_pmc = ["python3", bench, "--workload", name, "--profile-run", "--stream",
                    "--steps", "5", "--warmup", "2"]
    cmds = {}
    if prog:
        cmds["trace"] = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv",
                         "-d", os.path.join(out_dir, f"trace_{name}"), "-o", "trace", "--", *prog]
    for p, counters in PMC_PASSES.items():
        if name == "copy" and p == "sq":
            continue
        cmds[p] = ["rocprofv3", "--pmc", *counters, "--output-format", "csv",
                   "-d", os.path.join(out_dir, f"{p}_{name}"), "-o", p, "--", *prog_pmc]
    return cmds


def _show(cmd: list) -> str:
    """A command as it reads from the repository root (the profile summaries quote it)."""
    out = []
    for a in cmd:
        out.append(_rel(a) if os.path.isabs(a) and a.startswith(ROOT) else a)
    return " ".join(out)


def _csv_rows(path: str) -> list:
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(out_dir: str, pass_name: str, name: str, suffix: str) -> str:
    d = os.path.join(out_dir, f"{pass_name}_{name}")
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def _counters(out_dir: str, pass_name: str, name: str, kernel: str) -> tuple:
    """Per-dispatch values of each counter for kernels whose name contains `kernel`:
    ({counter: [values]}, kernel name)."""
    import collections
    vals, kname = collections.defaultdict(list), None
    for r in _csv_rows(_find(out_dir, pass_name, name, "counter_collection.csv")):
        if kernel in r["Kernel_Name"]:
            vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
            kname = r["Kernel_Name"]
    if not vals:
        raise ValueError(f"{pass_name}_{name}: no dispatch of {kernel}")
    return vals, kname


def _median(v):
    v = sorted(v)
    return v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])


def _record(path: str, tag: str) -> dict | None:
    if not os.path.exists(path):
        return None
    m = re.search(r"<!--\s*" + tag + r"\s+(\{.*?\})\s*-->", open(path).read(), re.S)
    return json.loads(m.group(1)) if m else None


def summarize_copy(out_dir: str, cmds: dict) -> str:
    """profiles/copy_calibration.md from the copy's fetch, write and read-request passes."""
    n = 1 << 29                                   # bf16 elements: 1 GiB read, 1 GiB written
    true_kib = 2 * n / 1024
    f, kname = _counters(out_dir, "fetch", "copy", COPY_KERNEL)
    w, _ = _counters(out_dir, "write", "copy", COPY_KERNEL)
    rq, _ = _counters(out_dir, "rdreq", "copy", COPY_KERNEL)
    fetch, write = _median(f["FETCH_SIZE"]), _median(w["WRITE_SIZE"])
    r128, r64 = _median(rq["TCC_EA0_RDREQ_128B_sum"]), _median(rq["TCC_EA0_RDREQ_64B_sum"])
    r32, rall = _median(rq["TCC_EA0_RDREQ_32B_sum"]), _median(rq["TCC_EA0_RDREQ_sum"])
    req_bytes = 128 * r128 + 64 * r64 + 32 * r32
    rec = {"fetch_factor": round(true_kib / fetch, 4), "write_factor": round(true_kib / write, 4)}
    # the copy's own bandwidth: the timed launches of its kernel trace (after the warm-up)
    tr = [r for r in _csv_rows(_find(out_dir, "trace", "copy", "kernel_trace.csv"))
          if COPY_KERNEL in r["Kernel_Name"]]
    tr.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in tr][-COPY_TRACE_STEPS:]
    avg_us = sum(dur) / len(dur)
    gbs = 4 * n / avg_us / 1e3
    text = f"""# HBM counter calibration with a plain copy kernel (MI355X)

Commands (repository root; `python3 bench.py --profile-workload copy` runs them and writes this
file):

""" + "".join(f"    {_show(c)}\n" for c in cmds.values()) + f"""
The copy is torch's elementwise kernel (`{kname[:60]}...`) negating a 2^29-element bf16 tensor
into another: 1 GiB read and 1 GiB written per launch.

| kernel trace (last {len(dur)} launches, after 5 warm-up ones) | value |
|---|---|
| average duration | {avg_us:.2f} us |
| achieved | {gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% of 8 TB/s) |
| min / max | {min(dur):.2f} / {max(dur):.2f} us |

A plain streaming kernel (torch's vectorized elementwise kernel, 8-element vectors, normal loads
and stores) on this box: a reference point for the prologue kernels, which stream with
non-temporal loads and stores (the stores at device scope in launches that write 128 MiB or
more).

| counter | per launch (median of {len(f['FETCH_SIZE'])}) | true | scale applied to kernel counters |
|---|---|---|---|
| FETCH_SIZE (KiB) | {fetch:.0f} | {true_kib:.0f} | {rec['fetch_factor']:.4f} |
| WRITE_SIZE (KiB) | {write:.0f} | {true_kib:.0f} | {rec['write_factor']:.4f} |

Why FETCH_SIZE reads half: its expression on this part is
`(TCC_BUBBLE*128 + (TCC_EA0_RDREQ - TCC_BUBBLE - TCC_EA0_RDREQ_32B)*64 + TCC_EA0_RDREQ_32B*32) / 1024`,
so a read request counts 64 bytes unless TCC_BUBBLE marks it as 128. The request-size counters of
the same copy:

| TCC_EA0_RDREQ | _128B | _64B | _32B | bytes from the sizes | true bytes | ratio |
|---|---|---|---|---|---|---|
| {rall:.0f} | {r128:.0f} | {r64:.0f} | {r32:.0f} | {req_bytes:,.0f} | {2 * n:,} | {req_bytes / (2 * n):.5f} |

Every read is a 128-byte request, which FETCH_SIZE counts as 64: the scale of 2 is the request
size, confirmed independently of the copy's known size. Each counter record of a prologue kernel
also gives its read bytes from the request sizes.

<!-- calibration {json.dumps(rec)} -->
"""
    path = os.path.join(ROOT, "profiles", "copy_calibration.md")
    open(path, "w").write(text)
    return path


def summarize_workload(name: str, out_dir: str, cmds: dict) -> list:
    """profiles/counters_NAME.md and profiles/sq_NAME.md from the passes' CSV files."""
    from qk_rmsnorm_rope_amd import workloads as wl
    w = wl.WORKLOADS[name]
    kern = kernel_name(w) + "<"
    cal = _record(os.path.join(ROOT, "profiles", "copy_calibration.md"), "calibration")
    if cal is None:
        raise RuntimeError("profile the copy first: bench.py --profile-workload copy")
    nbytes = algorithmic_bytes(w)
    # kernel trace: every dispatch, and the last 100 (bench.py's timed graph replay)
    tr = [r for r in _csv_rows(_find(out_dir, "trace", name, "kernel_trace.csv"))
          if kern in r["Kernel_Name"]]
    tr.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in tr]
    last = dur[-100:]
    gaps = [(int(b["Start_Timestamp"]) - int(a["End_Timestamp"])) / 1e3
            for a, b in zip(tr[-100:], tr[-99:])]
    srt = sorted(last)
    pct = lambda p: srt[min(len(srt) - 1, int(p * len(srt)))]
    avg, avg_last = sum(dur) / len(dur), sum(last) / len(last)
    k0 = tr[0]
    # bytes per dispatch
    f, _ = _counters(out_dir, "fetch", name, kern)
    wr, _ = _counters(out_dir, "write", name, kern)
    rq, _ = _counters(out_dir, "rdreq", name, kern)
    fetch_kib, write_kib = _median(f["FETCH_SIZE"]), _median(wr["WRITE_SIZE"])
    fetch_b = round(fetch_kib * 1024 * cal["fetch_factor"])
    write_b = round(write_kib * 1024 * cal["write_factor"])
    req_b = (128 * _median(rq["TCC_EA0_RDREQ_128B_sum"]) + 64 * _median(rq["TCC_EA0_RDREQ_64B_sum"])
             + 32 * _median(rq["TCC_EA0_RDREQ_32B_sum"]))
    read_alg, write_alg = nbytes - output_bytes(w), output_bytes(w)
    wr64 = _median(wr["TCC_EA0_WRREQ_64B_sum"]) if "TCC_EA0_WRREQ_64B_sum" in wr else 0.0
    wr32 = (_median(wr["TCC_EA0_WRREQ_sum"]) - wr64) if "TCC_EA0_WRREQ_sum" in wr else 0.0
    wr32_share = 32 * wr32 / max(32 * wr32 + 64 * wr64, 1)
    rec = {"bytes_per_launch": fetch_b + write_b, "fetch_bytes": fetch_b, "write_bytes": write_b,
           "read_request_bytes": round(req_b), "algorithmic_bytes": nbytes,
           "avg_kernel_us": round(avg, 2), "avg_kernel_us_last100": round(avg_last, 2),
           "kernel_source_hash": kernel_source_hash(w)}
    gb = lambda us: nbytes / (us * 1e-6) / 1e9
    pc = lambda us: gb(us) / PEAK_HBM_GBS
    shown = {p: _show(c) for p, c in cmds.items()}
    counters_md = f"""# {name}: rocprofv3 kernel trace and HBM counters (MI355X)

Commands (repository root; `python3 bench.py --profile-workload {name}` runs them and writes this
file and sq_{name}.md):

    {shown['trace']}
    {shown['fetch']}
    {shown['write']}
    {shown['rdreq']}

The kernel trace runs bench.py's own sequence (warm-up launches on the stream, then the 100 timed
steps captured in a HIP graph, replayed once to warm up and once timed); the counter passes
launch on the stream (per-dispatch counters do not depend on how the launch was submitted).

Kernel: `{k0['Kernel_Name']}`
(workgroup {k0['Workgroup_Size_X']}, grid {k0['Grid_Size_X']} work-items, LDS {k0['LDS_Block_Size']} B, scratch {k0['Scratch_Size']} B)

| kernel trace | value |
|---|---|
| dispatches | {len(dur)} |
| average duration | {avg:.2f} us |
| min / max | {min(dur):.2f} / {max(dur):.2f} us |
| algorithmic bytes per launch | {nbytes:,} |
| algorithmic GB/s at the average | {gb(avg):.0f} ({pc(avg):.1%} of 8 TB/s) |
| average of the last 100 (bench.py's timed graph replay) | {avg_last:.2f} us, {gb(avg_last):.0f} GB/s ({pc(avg_last):.1%} of 8 TB/s) |
| last 100: p10 / median / p90 | {pct(0.1):.2f} / {pct(0.5):.2f} / {pct(0.9):.2f} us (median: {pc(pct(0.5)):.1%} of 8 TB/s) |
| median idle gap between consecutive launches (last 100) | {_median(gaps) if gaps else 0.0:.2f} us |

| HBM bytes per dispatch (median of {len(f['FETCH_SIZE'])}) | raw | bytes | algorithmic bytes | ratio |
|---|---|---|---|---|
| FETCH_SIZE x {cal['fetch_factor']} | {fetch_kib:.0f} KiB | {fetch_b:,} | {read_alg:,} | {fetch_b / read_alg:.4f} |
| read requests x their size (128/64/32 B) | {_median(rq['TCC_EA0_RDREQ_sum']):.0f} requests | {req_b:,.0f} | {read_alg:,} | {req_b / read_alg:.4f} |
| WRITE_SIZE x {cal['write_factor']} | {write_kib:.0f} KiB | {write_b:,} | {write_alg:,} | {write_b / max(write_alg, 1):.4f} |

Write requests: {wr64:,.0f} of 64 bytes and {wr32:,.0f} of 32 bytes per dispatch ({wr32_share:.1%} of the written bytes
in 32-byte requests).

Calibration: profiles/copy_calibration.md. The record below is what bench.py reports as
`roofline.traffic` (FETCH_SIZE and WRITE_SIZE, calibrated); it is ignored once the kernel
sources hash differently.

<!-- traffic {json.dumps(rec)} -->
"""
    sq, _ = _counters(out_dir, "sq", name, kern)
    m = {c: _median(v) for c, v in sq.items()}
    sq_rows = [r for r in _csv_rows(_find(out_dir, "sq", name, "counter_collection.csv"))
               if kern in r["Kernel_Name"] and r["Counter_Name"] == "GRBM_GUI_ACTIVE"]
    dur_us = _median([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                      for r in sq_rows]) if sq_rows else 0.0
    cus, xcds = 256, 8
    try:
        info = _csv_rows(_find(out_dir, "sq", name, "agent_info.csv"))
        gpu = next(r for r in info if str(r.get("Name", "")).startswith("gfx"))
        cus, xcds = int(gpu["Cu_Count"]), int(gpu.get("Num_Xcc") or 1)
    except (FileNotFoundError, StopIteration, KeyError, ValueError):
        pass
    waves = m["SQ_WAVES"]
    # the per-dispatch GRBM_GUI_ACTIVE is summed over the XCDs, each counting its own busy
    # cycles; the derived metrics divide by one XCD's (rocprofv3 takes the maximum over them)
    active = m["GRBM_GUI_ACTIVE"] / xcds
    valu_busy = 100 * m["SQ_ACTIVE_INST_VALU"] / cus / active
    lds_conf = 100 * m["SQ_LDS_BANK_CONFLICT"] / cus / active
    sq_md = f"""# {name}: instruction mix and VALU / LDS use (rocprofv3 SQ counters, MI355X)

Command (repository root; written by `python3 bench.py --profile-workload {name}`):

    {shown['sq']}

Kernel `{k0['Kernel_Name']}`, medians over {len(sq['SQ_WAVES'])} dispatches of the stream-launched
sequence. VALU busy and LDS bank conflicts are rocprofv3's derived metrics VALUBusy =
100 * SQ_ACTIVE_INST_VALU / CU_NUM / GRBM_GUI_ACTIVE and LDSBankConflict =
100 * SQ_LDS_BANK_CONFLICT / GRBM_GUI_ACTIVE / CU_NUM, with CU_NUM = {cus} and GRBM_GUI_ACTIVE
one XCD's busy cycles (the recorded value is the sum over the {xcds} XCDs: {active:,.0f} cycles
each, {active / max(1e-9, dur_us):,.0f} MHz over the dispatch's {dur_us:.1f} us).

| counter (per dispatch) | value | per wave |
|---|---|---|
| SQ_WAVES | {waves:,.0f} | |
| SQ_INSTS_VALU | {m['SQ_INSTS_VALU']:,.0f} | {m['SQ_INSTS_VALU'] / waves:.1f} |
| SQ_INSTS_SALU | {m['SQ_INSTS_SALU']:,.0f} | {m['SQ_INSTS_SALU'] / waves:.1f} |
| SQ_INSTS_LDS | {m['SQ_INSTS_LDS']:,.0f} | {m['SQ_INSTS_LDS'] / waves:.1f} |
| SQ_LDS_BANK_CONFLICT (cycles) | {m['SQ_LDS_BANK_CONFLICT']:,.0f} | {m['SQ_LDS_BANK_CONFLICT'] / waves:.2f} |
| SQ_ACTIVE_INST_VALU | {m['SQ_ACTIVE_INST_VALU']:,.0f} | |
| GRBM_GUI_ACTIVE (cycles) | {m['GRBM_GUI_ACTIVE']:,.0f} | |
| **VALU busy** | **{valu_busy:.1f}%** | |
| LDS bank conflict | {lds_conf:.2f}% of cycles | |

<!-- sq {json.dumps({"valu_per_wave": round(m['SQ_INSTS_VALU'] / waves, 1), "valu_busy_pct": round(valu_busy, 1), "lds_bank_conflict_per_wave": round(m['SQ_LDS_BANK_CONFLICT'] / waves, 2), "kernel_source_hash": kernel_source_hash(w)})} -->
"""
    paths = []
    for fname, text in ((f"counters_{name}.md", counters_md), (f"sq_{name}.md", sq_md)):
        path = os.path.join(ROOT, "profiles", fname)
        open(path, "w").write(text)
        paths.append(path)
    return paths


def profile_workload(name: str, out_dir: str, only_summarize: bool = False) -> int:
    """Run the rocprofv3 passes of `name` (a workload, or "copy") as child processes, then
    write the summaries. Each pass prints one line; a pass that fails stops the run."""
    import subprocess
    out_dir = os.path.abspath(out_dir)
    os.makedirs(out_dir, exist_ok=True)
    cmds = profile_commands(name, out_dir)
    env = dict(os.environ, TMPDIR="/tmp")
    if not only_summarize:
        for p, cmd in cmds.items():
            t0 = time.time()
            log = os.path.join(out_dir, f"{p}_{name}.log")
            with open(log, "w") as lf:
                r = subprocess.run(cmd, cwd="/tmp", env=env, stdout=lf, stderr=subprocess.STDOUT,
                                   timeout=300)
            print(f"profile {name} {p}: rc {r.returncode} in {time.time() - t0:.1f}s", flush=True)
            # rocprofv3 itself may end with a segmentation fault after the program is done and
            # its output written; the summary below checks that the files are there
            if r.returncode not in (0, -11, 139):
                print(open(log).read()[-3000:], flush=True)
                return r.returncode
    paths = summarize_copy(out_dir, cmds) if name == "copy" else \
        summarize_workload(name, out_dir, cmds)
    for p in ([paths] if isinstance(paths, str) else paths):
        print(f"wrote {_rel(p)}", flush=True)
    return 0


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
    ap.add_argument("--profile-workload", metavar="NAME",
                    help="run the rocprofv3 passes of NAME (a workload, or 'copy') and write "
                         "its summaries under profiles/")
    ap.add_argument("--profile-dir", default=os.path.join(ROOT, "gpurun_out", "prof"),
                    help="where --profile-workload keeps rocprofv3's raw output")
    ap.add_argument("--summarize-only", action="store_true",
                    help="with --profile-workload: rewrite the summaries from existing output")
    args = ap.parse_args()
    if args.profile_workload:
        return profile_workload(args.profile_workload, args.profile_dir, args.summarize_only)

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
