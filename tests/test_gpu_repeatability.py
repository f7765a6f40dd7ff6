"""Repeatability on the GPU: the same call, launched many times into outputs refilled with a
marker pattern in between, writes every output byte, and writes the same bytes every time.

The kernels take no atomics and reduce in a fixed order (DPP/permlane trees, one LDS pass), so
any difference between two launches would mean a race, a read of memory no lane wrote, or a
missing wait; the parity tests compare against the oracle within a tolerance and would not see a
difference of an ulp between launches. Shapes: the two large across-heads 3D workloads at full
size (one and two tokens per workgroup, bf16 and E4M3 outputs), a 13-wave mixed-slot 3D shape
with NeoX pairs (10/17/22 heads of 128), the 4096-token table form, the camera prologue at full
size, and one rank's two-kernel step of a head-sharded run.
"""
from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu

qr = pytest.importorskip("qk_rmsnorm_rope_amd")
from qk_rmsnorm_rope_amd import workloads as wl  # noqa: E402

DEV = "cuda"

MIXED_NEOX = wl.Rope3DWorkload(
    name="mixed_neox_t50_h10_17_22_d128", batch=2, ppf=5, pph=1, ppw=5,
    num_frame_channels=82, num_height_channels=36, num_width_channels=10, num_heads_q=10,
    num_heads_k=17, num_heads_v=22, head_dim=128, seed=9352, eps=1e-3, base=1e4,
    interleave=False, is_qk_norm=True, sigma=3.0)


def _repeat(call, outs, reps):
    call()
    torch.cuda.synchronize()
    first = [o.view(torch.uint8).clone() for o in outs]
    for k in range(reps):
        for o in outs:
            o.view(torch.uint8).fill_(0x5A if k % 2 else 0xA5)
        call()
        for r, (o, f) in enumerate(zip(outs, first)):
            if not torch.equal(o.view(torch.uint8), f):
                n = int((o.view(torch.uint8) != f).sum())
                raise AssertionError(f"launch {k + 1}, output {r}: {n} bytes differ from launch 0")


@pytest.mark.parametrize("name,reps", [("rope3d_across_interleaved_s15360_h32_d128", 300),
                                       ("rope3d_neox_fp8_b2_s18480_h20_d64", 300),
                                       ("mixed_neox", 3000)])
def test_3d_launches_repeat_bit_for_bit(name, reps):
    w = MIXED_NEOX if name == "mixed_neox" else wl.WORKLOADS[name]
    inp = wl.rope3d_inputs(w)
    qkv, wq, wk = (inp[k].to(DEV) for k in ("qkv", "q_weight", "k_weight"))
    odt = torch.float8_e4m3fn if w.output_fp8 else torch.bfloat16
    outs = [torch.empty((w.num_tokens, h, w.head_dim), dtype=odt, device=DEV)
            for h in (w.num_heads_q, w.num_heads_k, w.num_heads_v)]
    _repeat(qr.Prepared3D(w, qkv, wq, wk, *outs), outs, reps)


def test_table_launches_repeat_bit_for_bit():
    w = wl.WORKLOADS["table_interleaved_t4096_h24_d128_bf16table"]
    g = {k: v.to(DEV) for k, v in wl.table_inputs(w).items()}
    qo, ko = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    call = qr.PreparedTable(g["q"], g["k"], g["q_weight"], g["k_weight"], g["rope_table"], w.eps,
                            q_out=qo, k_out=ko, rotary_dim=w.rotary_dim,
                            interleaved=w.interleaved, norm_mode=w.norm_mode,
                            out_scale=w.out_scale)
    _repeat(call, [qo, ko], 1000)


def test_camera_prologue_launches_repeat_bit_for_bit():
    w = wl.WORKLOADS["cam_prep_b2_s18480_h20_d64"]
    g = {k: v.to(DEV) for k, v in wl.cam_inputs(w).items()}
    B, N, H, D = w.batch, w.num_tokens, w.num_heads, w.head_dim
    outs = [torch.empty((B, H, D, N), dtype=g["q"].dtype, device=DEV) for _ in range(3)]
    infl = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    call = qr.PreparedCam(g["q"], g["k"], g["v"], g["proj_q"], g["proj_kv"], g["rope_cos"],
                          g["rope_sin"], w.k_scale, *outs, infl)
    _repeat(call, outs + [infl], 300)


def test_head_sharded_step_repeats_bit_for_bit():
    """The two-kernel step of one head shard: per-token sums of squares, then the apply kernel
    normalising with them (sums and outputs both compared)."""
    w = wl.WORKLOADS["rope3d_across_interleaved_s15360_h32_d128_tp4rank"]
    g = {k: v.to(DEV) for k, v in wl.rope3d_inputs(w).items()}
    outs = [torch.empty((w.num_tokens, h, w.head_dim), dtype=torch.bfloat16, device=DEV)
            for h in (w.num_heads_q, w.num_heads_k, w.num_heads_v)]
    ss = torch.empty((w.num_tokens, 2), dtype=torch.float32, device=DEV)
    call = qr.PreparedSharded3D(w, g["qkv"], g["q_weight"], g["k_weight"], *outs, ss, ss)
    _repeat(call, outs + [ss], 300)
