"""The largest head counts one workgroup per token covers, against the fp64 oracle, and the first
ones past them refused.

A lane holds at most eight 16-byte chunks of a token, so with 1024-lane workgroups the 3D form
takes up to 2048 chunks (heads x head_dim / 8) in each of Q, K and V with two slots per region,
or up to 4096 in all three together with four mixed slots; the table form up to 4096 lane units
(heads x head_dim / 8 rounded up to a power of two) in each of Q and K with four slots. These
cases run the widest slot layouts at 1024 lanes.
"""
from __future__ import annotations

import pytest
import torch

import oracle
from parity import check_3d_outputs, check_table_outputs

pytestmark = pytest.mark.gpu

qr = pytest.importorskip("qk_rmsnorm_rope_amd")
from qk_rmsnorm_rope_amd import workloads as wl  # noqa: E402

DEV = "cuda"


def rope3d(D, hq, hk, hv, seed, **kw):
    c = D // 4
    return wl.Rope3DWorkload(name=f"limit3d_d{D}_{hq}-{hk}-{hv}", batch=2, ppf=1, pph=2, ppw=4,
                             num_frame_channels=D - 2 * c, num_height_channels=c,
                             num_width_channels=c, num_heads_q=hq, num_heads_k=hk,
                             num_heads_v=hv, head_dim=D, seed=seed, **kw)


@pytest.mark.parametrize("w", [
    rope3d(128, 128, 128, 128, wl.SEED_BASE + 400),                       # 2048 chunks a region
    rope3d(256, 64, 64, 64, wl.SEED_BASE + 401, interleave=False, output_fp8=True,
           output_quant_scale=0.5, v_quant_scale=0.25),
    rope3d(128, 256, 0, 0, wl.SEED_BASE + 402),                           # 4096 chunks, Q only
    rope3d(64, 200, 150, 160, wl.SEED_BASE + 403, is_qk_norm=False),      # uneven, <= 2048 each
], ids=lambda w: w.name)
def test_3d_largest_rows(w):
    print(f"\n{w.name}: {w.num_tokens} tokens, row {w.row_elems}", flush=True)
    inp = wl.rope3d_inputs(w)
    qkv, wq, wk = (inp[k].to(DEV) for k in ("qkv", "q_weight", "k_weight"))
    outs = qr.run_workload_3d(w, qkv, wq, wk)
    torch.cuda.synchronize()
    ref = oracle.run_3d_workload(w, inp["qkv"].reshape(-1, w.row_elems), inp["q_weight"],
                                 inp["k_weight"])
    check_3d_outputs(w, outs, ref)


@pytest.mark.parametrize("heads", [(129, 128, 128), (257, 0, 0), (1, 1, 4097)])
def test_3d_past_the_largest_rows_is_unsupported(heads):
    w = rope3d(128, *heads, seed=1).with_(batch=1)
    qkv = torch.zeros((w.num_tokens, w.row_elems), dtype=torch.bfloat16, device=DEV)
    wq = torch.ones(max(1, heads[0]) * 128, dtype=torch.bfloat16, device=DEV)
    wk = torch.ones(max(1, heads[1]) * 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="too many heads"):
        qr.run_workload_3d(w, qkv, wq, wk)


@pytest.mark.parametrize("inter,norm,D,H", [(True, "per_head", 128, 256),
                                            (False, "across_heads", 256, 128)])
def test_table_largest_rows(inter, norm, D, H):
    w = wl.TableWorkload(name=f"limit_table_d{D}_h{H}", num_tokens=9, num_heads_q=H,
                         num_heads_k=H, head_dim=D, rotary_dim=D, interleaved=inter,
                         table_dtype="f32", seed=wl.SEED_BASE + 410 + H, norm_mode=norm)
    inp = wl.table_inputs(w)
    g = {k: v.to(DEV) for k, v in inp.items()}
    qo, ko = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    qr.qkrope_run_table(g["q"], g["k"], g["q_weight"], g["k_weight"], g["rope_table"], w.eps,
                        q_out=qo, k_out=ko, rotary_dim=D, interleaved=inter, norm_mode=norm)
    torch.cuda.synchronize()
    rq, rk = oracle.run_table(inp["q"], inp["k"], inp["q_weight"], inp["k_weight"],
                              inp["rope_table"], w.eps, rotary_dim=D, interleaved=inter,
                              norm_mode=norm)
    check_table_outputs(w.name, qo, ko, rq, rk)


def test_table_past_the_largest_rows_is_unsupported():
    q = torch.zeros((2, 257, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((2, 1, 128), dtype=torch.bfloat16, device=DEV)
    w1 = torch.ones(128, dtype=torch.bfloat16, device=DEV)
    tab = torch.zeros((2, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError, match="too many heads"):
        qr.qkrope_run_table(q, k, w1, w1, tab, 1e-6, q_out=torch.empty_like(q),
                            k_out=torch.empty_like(k))
