"""Seeded random sweep over the whole contract, on the GPU, against the fp64 oracle.

Each case draws a valid argument set (head counts from 0 up, head_dim, channel split, grid,
pairing, norm, YaRN, FP8 and its scales for the 3D form; head_dim, rotary_dim from 0, pairing,
norm, activation and table formats, split tables with padded strides, strided inputs, E4M3 or
16-bit outputs, in-place use for the table form) and compares every output element with the
oracle at the usual criteria. It exists to reach launch shapes and code paths that the
hand-written cases do not name (slot layouts, two tokens per workgroup, LDS partner exchange,
scalar and vector table reads).
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle
from parity import (assert_bf16_close, assert_e4m3_within_one, assert_f16_close,
                    check_3d_outputs)

pytestmark = pytest.mark.gpu

qr = pytest.importorskip("qk_rmsnorm_rope_amd")
from qk_rmsnorm_rope_amd import workloads as wl  # noqa: E402

DEV = "cuda"
# cases per form; QKROPE_SWEEP_CASES runs that many of each instead (same draws, more indices)
N3D = NTAB = int(os.environ.get("QKROPE_SWEEP_CASES", "400"))
# 3D cases (every fourth below this) that also run as two sequence shards, checked bit for bit
N_SHARD = 80


def describe_mismatch(got, want, t0, label):
    """Where two [tokens, heads, head_dim] outputs differ (tokens offset by t0), and whether
    the difference is still there when compared again."""
    g, wv = got.view(torch.uint8), want.view(torch.uint8)
    d = (g != wv).nonzero().cpu()
    toks = sorted({int(x) + t0 for x in d[:, 0]})
    heads = sorted({int(x) for x in d[:, 1]})
    t, h, e = (int(x) for x in d[0])
    torch.cuda.synchronize()
    again = torch.equal(g, wv)
    return (f"{label}: {len(d)} bytes differ at tokens {toks[:16]} heads {heads[:24]}; first at "
            f"token {t + t0} head {h} byte {e}: {int(g[t, h, e])} vs {int(wv[t, h, e])}; "
            f"equal when compared again: {again}")


def pow2_on_even(i, v):
    """Even cases round their V scale to the nearest power of two, where V's E4M3 codes take the
    scaled packed conversion and must equal the oracle's bit for bit; odd cases keep the drawn
    scale (the general path). The draw itself is unchanged, so the other draws keep their order."""
    return float(2.0 ** round(math.log2(v))) if i % 2 == 0 else v


def draw_3d(i):
    rng = np.random.default_rng(9000 + i)
    D = int(rng.choice([64, 128, 256]))
    H = [int(x) for x in rng.integers(0, 41, 3)]
    if sum(H) == 0:
        H[0] = 1
    cf = 2 * int(rng.integers(0, D // 2 + 1))
    ch = 2 * int(rng.integers(0, (D - cf) // 2 + 1))
    cw = D - cf - ch
    grid = [int(x) for x in rng.integers(1, 7, 3)]
    batch = int(rng.integers(1, 4))
    yarn = bool(rng.random() < 0.4)
    low = float(rng.uniform(-2, 8)) if yarn else 0.0
    fp8 = bool(rng.random() < 0.4)
    return wl.Rope3DWorkload(
        name=f"rand3d_{i}", batch=batch, ppf=grid[0], pph=grid[1], ppw=grid[2],
        num_frame_channels=cf, num_height_channels=ch, num_width_channels=cw,
        num_heads_q=H[0], num_heads_k=H[1], num_heads_v=H[2], head_dim=D, seed=9100 + i,
        eps=float(rng.choice([1e-6, 1e-5, 1e-3])), base=float(rng.choice([1e4, 500.0, 1e6])),
        interleave=bool(rng.random() < 0.5),
        factor=float(rng.uniform(1.5, 8)) if yarn else 1.0, low=low,
        high=low + float(rng.uniform(0.5, 30)) if yarn else 0.0,
        attention_factor=float(rng.uniform(0.8, 1.3)) if yarn else 1.0,
        is_qk_norm=bool(rng.random() < 0.7), output_fp8=fp8,
        output_quant_scale=float(rng.uniform(0.1, 4)) if fp8 else 1.0,
        v_quant_scale=pow2_on_even(i, float(rng.uniform(0.1, 4))) if fp8 else 1.0,
        sigma=float(rng.choice([1.0, 3.0])))


@pytest.mark.parametrize("i", range(N3D))
def test_random_3d(i):
    w = draw_3d(i)
    inp = wl.rope3d_inputs(w)
    qkv, wq, wk = (inp[k].to(DEV) for k in ("qkv", "q_weight", "k_weight"))
    outs = qr.run_workload_3d(w, qkv, wq, wk)
    torch.cuda.synchronize()
    ref = oracle.run_3d_workload(w, inp["qkv"].reshape(-1, w.row_elems), inp["q_weight"],
                                 inp["k_weight"])
    check_3d_outputs(w, outs, ref)
    if i % 4 == 0 and i < N_SHARD and w.num_tokens > 2:
        # the same tokens as two sequence shards give the same bits
        rng = np.random.default_rng(9200 + i)
        cut = int(rng.integers(1, w.num_tokens))
        x = qkv.reshape(w.num_tokens, -1)
        odt = torch.float8_e4m3fn if w.output_fp8 else torch.bfloat16
        kw = dict(ppf=w.ppf, pph=w.pph, ppw=w.ppw, num_frame_channels=w.num_frame_channels,
                  num_height_channels=w.num_height_channels,
                  num_width_channels=w.num_width_channels, num_heads_q=w.num_heads_q,
                  num_heads_k=w.num_heads_k, num_heads_v=w.num_heads_v, head_dim=w.head_dim,
                  eps=w.eps, base=w.base, interleave=w.interleave, factor=w.factor, low=w.low,
                  high=w.high, attention_factor=w.attention_factor, is_qk_norm=w.is_qk_norm,
                  output_fp8=w.output_fp8, output_quant_scale=w.output_quant_scale,
                  v_quant_scale=w.v_quant_scale)
        for a, b in ((0, cut), (cut, w.num_tokens)):
            o = [torch.empty((b - a, H, w.head_dim), dtype=odt, device=DEV)
                 for H in (w.num_heads_q, w.num_heads_k, w.num_heads_v)]
            qr.qkrope_run_3d_sharded(x[a:b].contiguous(), wq, wk, token_offset=a, q_out=o[0],
                                     k_out=o[1], v_out=o[2], **kw)
            torch.cuda.synchronize()
            for r in range(3):
                full = outs[r].reshape(w.num_tokens, -1, w.head_dim)[a:b]
                assert torch.equal(o[r].view(torch.uint8), full.view(torch.uint8)), \
                    describe_mismatch(o[r], full, a, (a, b, r))


def draw_table(i):
    rng = np.random.default_rng(7000 + i)
    D = 8 * int(rng.integers(1, 33))
    R = 2 * int(rng.integers(0, D // 2 + 1))
    act = "f16" if rng.random() < 0.4 else "bf16"
    tdt = "f32" if rng.random() < 0.5 else act
    mode = str(rng.choice(["per_head", "per_head", "across_heads", "none"]))
    e4m3 = bool(rng.random() < 0.3)
    return dict(T=int(rng.integers(1, 201)), Hq=int(rng.integers(0, 49)),
                Hk=int(rng.integers(0, 49)), D=D, R=R, interleaved=bool(rng.random() < 0.5),
                mode=mode, act=act, tdt=tdt, e4m3=e4m3,
                scale=float(rng.uniform(0.1, 4)) if e4m3 else 1.0,
                split=bool(rng.random() < 0.5), pad=8 * int(rng.integers(0, 3)),
                inplace=bool(not e4m3 and rng.random() < 0.3),
                sigma=float(rng.choice([1.0, 3.0])))


@pytest.mark.parametrize("i", range(NTAB))
def test_random_table(i):
    c = draw_table(i)
    if c["Hq"] + c["Hk"] == 0:
        c["Hq"] = 1
    w = wl.TableWorkload(name=f"randtab_{i}", num_tokens=c["T"], num_heads_q=c["Hq"],
                         num_heads_k=c["Hk"], head_dim=c["D"], rotary_dim=c["R"],
                         interleaved=c["interleaved"], table_dtype=c["tdt"], seed=7100 + i,
                         norm_mode=c["mode"], act_dtype=c["act"], sigma=c["sigma"])
    inp = wl.table_inputs(w)
    T, Hq, Hk, D, R, pad = c["T"], c["Hq"], c["Hk"], c["D"], c["R"], c["pad"]
    dt = inp["q"].dtype
    # q and k as views of one padded token row; the table either packed or split, padded
    packed = torch.zeros(T, (Hq + Hk) * D + pad, dtype=dt, device=DEV)
    packed[:, :Hq * D] = inp["q"].to(DEV).reshape(T, -1)
    packed[:, Hq * D:(Hq + Hk) * D] = inp["k"].to(DEV).reshape(T, -1)
    q = packed[:, :Hq * D].view(T, Hq, D)
    k = packed[:, Hq * D:(Hq + Hk) * D].view(T, Hk, D)
    tab = inp["rope_table"].to(DEV)
    if c["split"]:
        cbuf = torch.zeros(T, R // 2 + pad + 2, dtype=tab.dtype, device=DEV)
        sbuf = torch.zeros(T, R // 2 + 2 * pad + 4, dtype=tab.dtype, device=DEV)
        cbuf[:, : R // 2] = tab[:, : R // 2]
        sbuf[:, : R // 2] = tab[:, R // 2: R]
        cos_t, sin_t = cbuf[:, : R // 2], sbuf[:, : R // 2]
    else:
        cos_t, sin_t = tab[:, : R // 2], tab[:, R // 2: R]
    wq, wk = inp["q_weight"].to(DEV), inp["k_weight"].to(DEV)
    if c["inplace"]:
        qo, ko = q, k
    else:
        odt = torch.float8_e4m3fn if c["e4m3"] else dt
        qo = torch.empty((T, Hq, D), dtype=odt, device=DEV)
        ko = torch.empty((T, Hk, D), dtype=odt, device=DEV)
    rq, rk = oracle.run_table(inp["q"], inp["k"], inp["q_weight"], inp["k_weight"],
                              inp["rope_table"], w.eps, rotary_dim=R,
                              interleaved=c["interleaved"], norm_mode=c["mode"])
    qr.qkrope_run_table_ex(q, k, wq, wk, cos_t, sin_t, w.eps, q_out=qo, k_out=ko, head_dim=D,
                           rotary_dim=R, interleaved=c["interleaved"], norm_mode=c["mode"],
                           out_scale=c["scale"])
    torch.cuda.synchronize()
    for name, o, r in (("q", qo, rq), ("k", ko, rk)):
        if r.size == 0:
            continue
        if c["e4m3"]:
            assert_e4m3_within_one(o, oracle.e4m3_encode(r, c["scale"]), f"{c} {name}")
        elif c["act"] == "f16":
            assert_f16_close(o, r, f"{c} {name}")
        else:
            assert_bf16_close(o, r, f"{c} {name}")
