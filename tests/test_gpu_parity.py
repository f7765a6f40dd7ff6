"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by element.

Sizes: each named workload at a size the oracle finishes in seconds (several workgroups' worth of
tokens, ragged where the shape allows), the 3D workloads at full size at every token, and a
seeded sweep over the contract's parameters (pairing, norm mode, YaRN, FP8, head counts, tiny and
degenerate grids, strided and in-place table views).
"""
from __future__ import annotations


import numpy as np
import pytest
import torch

import oracle
from parity import (assert_bf16_close, assert_bits_equal, assert_e4m3_within_one,
                    check_3d_outputs, check_table_outputs)

pytestmark = pytest.mark.gpu

qr = pytest.importorskip("qk_rmsnorm_rope_amd")
from qk_rmsnorm_rope_amd import workloads as wl  # noqa: E402

DEV = "cuda"


def _gpu(t):
    return t.to(DEV)


def run_3d(w, inputs):
    qkv, wq, wk = (_gpu(inputs[k]) for k in ("qkv", "q_weight", "k_weight"))
    outs = qr.run_workload_3d(w, qkv, wq, wk)
    torch.cuda.synchronize()
    return outs


def oracle_3d(w, inputs):
    x = inputs["qkv"].reshape(-1, w.row_elems)
    return oracle.run_3d_workload(w, x, inputs["q_weight"], inputs["k_weight"])


def run_table(w, inputs, **kw):
    q, k, wq, wk, tab = (_gpu(inputs[n]) for n in ("q", "k", "q_weight", "k_weight", "rope_table"))
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    qr.qkrope_run_table(q, k, wq, wk, tab, w.eps, q_out=qo, k_out=ko, rotary_dim=w.rotary_dim,
                        interleaved=w.interleaved, norm_mode=w.norm_mode, **kw)
    torch.cuda.synchronize()
    return qo, ko


def oracle_table(w, inputs):
    return oracle.run_table(inputs["q"], inputs["k"], inputs["q_weight"], inputs["k_weight"],
                            inputs["rope_table"], w.eps, rotary_dim=w.rotary_dim,
                            interleaved=w.interleaved, norm_mode=w.norm_mode)


# --- the named workloads, reduced so the oracle runs in seconds ---------------------------------

REDUCED_3D = [
    wl.ROPE3D_ACROSS_S15360.with_(ppf=2),                   # 1920 tokens, positions f in {0,1}
    wl.ROPE3D_NEOX_FP8_S18480.with_(ppf=2, pph=7),          # batch 2 x 392 tokens
    wl.ROPE3D_YARN_S122880.with_(ppf=1, pph=9),             # 720 tokens
]


@pytest.mark.parametrize("w", REDUCED_3D, ids=lambda w: w.name)
def test_3d_workload_reduced(w):
    inputs = wl.rope3d_inputs(w)
    outs = run_3d(w, inputs)
    check_3d_outputs(w, outs, oracle_3d(w, inputs))


@pytest.mark.parametrize("w", [wl.TABLE_HALFSPLIT_T256, wl.TABLE_INTERLEAVED_T4096],
                         ids=lambda w: w.name)
def test_table_workload_full(w):
    inputs = wl.table_inputs(w)
    qo, ko = run_table(w, inputs)
    rq, rk = oracle_table(w, inputs)
    check_table_outputs(w.name, qo, ko, rq, rk)


def test_table_workload_ragged_tokens():
    w = wl.TABLE_INTERLEAVED_T4096.with_(num_tokens=333)
    inputs = wl.table_inputs(w)
    qo, ko = run_table(w, inputs)
    check_table_outputs(w.name, qo, ko, *oracle_table(w, inputs))


# --- the named 3D workloads at full size, every token -------------------------------------------

FULL_CHUNK = 8192


@pytest.mark.timeout(600)
@pytest.mark.parametrize("w", [wl.ROPE3D_ACROSS_S15360, wl.ROPE3D_NEOX_FP8_S18480,
                               wl.ROPE3D_YARN_S122880], ids=lambda w: w.name)
def test_3d_workload_full_size_every_token(w):
    """One launch over the whole workload, every output element checked: the oracle runs over
    consecutive token chunks, each given its first token's index as the offset (positions
    (offset + t) mod S, so a chunk may cross a sequence boundary)."""
    inputs = wl.rope3d_inputs(w)
    outs = run_3d(w, inputs)
    x = inputs["qkv"].reshape(-1, w.row_elems)
    for a in range(0, w.num_tokens, FULL_CHUNK):
        b = min(w.num_tokens, a + FULL_CHUNK)
        ref = oracle.run_3d_workload(w, x[a:b], inputs["q_weight"], inputs["k_weight"],
                                     token_offset=a)
        check_3d_outputs(w, outs, ref, tokens=np.arange(a, b))


# --- seeded sweep over the 3D contract ----------------------------------------------------------

SWEEP_3D = [
    # (D, Hq, Hk, Hv, grid, channels, batch, interleave, norm, fp8, yarn)
    (64, 3, 2, 5, (2, 3, 4), (16, 24, 24), 2, True, True, False, False),
    (64, 1, 1, 1, (1, 1, 1), (0, 0, 64), 3, False, True, True, False),
    (128, 4, 4, 4, (3, 1, 5), (32, 48, 48), 1, False, False, False, True),
    (128, 6, 2, 1, (1, 4, 1), (16, 56, 56), 2, True, True, True, True),
    (256, 2, 3, 2, (2, 2, 2), (64, 96, 96), 1, True, False, True, True),
    (256, 5, 5, 5, (1, 2, 7), (0, 128, 128), 1, False, True, False, False),
    (128, 32, 32, 32, (1, 2, 3), (16, 56, 56), 2, True, True, False, False),
    (64, 20, 20, 20, (2, 3, 2), (16, 24, 24), 1, True, True, True, False),
    (128, 8, 0, 8, (1, 1, 4), (128, 0, 0), 1, True, True, False, False),
    # two tokens per workgroup (160 lanes a token), odd token count: the last workgroup has one
    (64, 20, 20, 20, (1, 3, 5), (16, 24, 24), 1, False, True, True, False),
    (128, 10, 6, 10, (1, 1, 7), (32, 48, 48), 1, True, True, False, True),
    # head_dim 256 with few heads: fewer chunk lanes per token than angle pairs (128)
    (256, 1, 1, 0, (1, 2, 3), (64, 96, 96), 1, True, True, False, True),
    (256, 2, 2, 2, (2, 1, 3), (64, 96, 96), 1, False, True, True, False),
    (256, 2, 0, 0, (1, 1, 5), (0, 128, 128), 1, False, False, True, False),
]


@pytest.mark.parametrize("case", SWEEP_3D, ids=lambda c: "d{}_h{}-{}-{}_g{}".format(c[0], *c[1:4], "x".join(map(str, c[4]))))
def test_3d_sweep(case):
    D, Hq, Hk, Hv, (f, h, ww), (cf, ch, cw), B, inter, norm, fp8, yarn = case
    w = wl.Rope3DWorkload(
        name=f"sweep_d{D}", batch=B, ppf=f, pph=h, ppw=ww, num_frame_channels=cf,
        num_height_channels=ch, num_width_channels=cw, num_heads_q=Hq, num_heads_k=Hk,
        num_heads_v=Hv, head_dim=D, seed=1000 + D + Hq, interleave=inter, is_qk_norm=norm,
        output_fp8=fp8, output_quant_scale=0.75 if fp8 else 1.0,
        v_quant_scale=0.5 if fp8 else 1.0, sigma=3.0 if fp8 else 1.0,
        factor=2.0 if yarn else 1.0, low=0.5 if yarn else 0.0, high=6.0 if yarn else 0.0,
        attention_factor=1.07 if yarn else 1.0, base=500.0 if yarn else 10000.0)
    inputs = wl.rope3d_inputs(w)
    check_3d_outputs(w, run_3d(w, inputs), oracle_3d(w, inputs))


def test_3d_fp8_saturation_and_non_power_of_two_v_scale():
    w = wl.ROPE3D_NEOX_FP8_S18480.with_(ppf=1, pph=2, ppw=4, batch=1, sigma=300.0,
                                       output_quant_scale=3.0, v_quant_scale=1.7)
    inputs = wl.rope3d_inputs(w)
    check_3d_outputs(w, run_3d(w, inputs), oracle_3d(w, inputs))


@pytest.mark.parametrize("v_scale", [0.125, 0.25, 4.0])
def test_3d_fp8_v_power_of_two_scale_edges(v_scale):
    """E4M3 of V with a power-of-two scale is exact scaling then one rounding, so its codes must
    equal the oracle's bit for bit, also where they saturate (sigma 300 puts many values past
    448 / s at s = 4, few at s = 0.125) and at planted infinities, zeros, the limit 448 / s
    itself, the next bf16 value above it, the smallest subnormal result and a rounding tie
    between subnormal codes."""
    w = wl.ROPE3D_NEOX_FP8_S18480.with_(ppf=1, pph=2, ppw=4, batch=2, sigma=300.0,
                                       output_quant_scale=0.5, v_quant_scale=v_scale)
    inputs = wl.rope3d_inputs(w)
    x = inputs["qkv"].reshape(w.num_tokens, w.row_elems).clone()
    lim = 448.0 / v_scale
    above = torch.tensor([lim], dtype=torch.bfloat16).view(torch.int16) + 1
    edge = torch.tensor([float("inf"), float("-inf"), 0.0, -0.0, lim, -lim,
                         2.0 ** -9 / v_scale, 1.5 * 2.0 ** -9 / v_scale], dtype=torch.bfloat16)
    voff = (w.num_heads_q + w.num_heads_k) * w.head_dim
    x[0, voff:voff + 8] = edge                                   # one chunk over the limit (inf)
    x[1, voff:voff + 8] = edge[2:].repeat(2)[:8]                 # within it: fast path, at lim
    x[2, voff + 8:voff + 16] = above.view(torch.bfloat16).repeat(8)   # just above the limit
    x[3, voff:voff + 8] = (edge[6:8] * 3).repeat(4)             # small codes only
    inputs["qkv"] = x.reshape(inputs["qkv"].shape)
    check_3d_outputs(w, run_3d(w, inputs), oracle_3d(w, inputs))


@pytest.mark.parametrize("fp8", [False, True])
def test_3d_nan_inputs_propagate(fp8):
    """A NaN in a token's K row makes its across-heads norm NaN, so every K output of that token
    is NaN (E4M3: the NaN code); a NaN in V stays in its own element; every other token and
    element matches the oracle as usual."""
    w = wl.ROPE3D_NEOX_FP8_S18480.with_(ppf=1, pph=2, ppw=4, batch=2, output_fp8=fp8)
    inputs = wl.rope3d_inputs(w)
    x = inputs["qkv"].reshape(w.num_tokens, w.row_elems).clone()
    D, Hq, Hk = w.head_dim, w.num_heads_q, w.num_heads_k
    x[3, Hq * D + 5] = float("nan")                         # token 3, K
    x[6, (Hq + Hk) * D + 17] = float("nan")                 # token 6, V element 17
    inputs["qkv"] = x.reshape(inputs["qkv"].shape)
    outs = [o.reshape(w.num_tokens, -1) for o in run_3d(w, inputs)]
    ref = oracle_3d(w, inputs)

    def is_nan(o):
        if fp8:
            return (o.view(torch.uint8).cpu() & 0x7F) == 0x7F
        return torch.isnan(o.float().cpu())

    assert bool(is_nan(outs[1][3]).all()), "every K output of the NaN token"
    v_nan = is_nan(outs[2][6])
    assert bool(v_nan[17]) and int(v_nan.sum()) == 1, "V: only the NaN element"
    assert not bool(is_nan(outs[0]).any()), "Q has no NaN"
    keep = [t for t in range(w.num_tokens) if t not in (3, 6)]
    check = [o[keep] for o in outs]
    refs = [r.reshape(w.num_tokens, -1)[keep] for r in ref]
    names = ("q", "k", "v")
    for i in range(3):
        if fp8:
            scale = w.v_quant_scale if i == 2 else w.output_quant_scale
            codes = oracle.e4m3_encode(refs[i], scale)
            (assert_bits_equal if i == 2 else assert_e4m3_within_one)(check[i], codes, names[i])
        elif i == 2:
            assert_bits_equal(check[i], oracle.bf16_encode(refs[i]), names[i])
        else:
            assert_bf16_close(check[i], refs[i], names[i])


@pytest.mark.parametrize("fp8", [False, True])
def test_3d_zero_rows(fp8):
    """Rows of zeros are a degenerate case of the norm (mean of squares 0, scale eps^-1/2): their
    outputs are zeros, exactly as the oracle's, in both output formats."""
    w = wl.ROPE3D_ACROSS_S15360.with_(ppf=1, pph=2, ppw=4, batch=2, output_fp8=fp8,
                                     output_quant_scale=0.5, v_quant_scale=0.25)
    inputs = wl.rope3d_inputs(w)
    x = inputs["qkv"].reshape(w.num_tokens, w.row_elems).clone()
    qd, kd = w.num_heads_q * w.head_dim, w.num_heads_k * w.head_dim
    x[2, :qd] = 0                         # token 2: Q row
    x[5, qd:qd + kd] = 0                  # token 5: K row
    x[7] = 0                              # token 7: everything
    inputs["qkv"] = x.reshape(inputs["qkv"].shape)
    outs = run_3d(w, inputs)
    check_3d_outputs(w, outs, oracle_3d(w, inputs))
    flat = [o.reshape(w.num_tokens, -1).view(torch.uint8 if fp8 else torch.int16) for o in outs]
    zero = 0
    assert bool((flat[0][2] & (0x7F if fp8 else 0x7FFF) == zero).all())
    assert bool((flat[1][5] & (0x7F if fp8 else 0x7FFF) == zero).all())
    assert all(bool((f[7] & (0x7F if fp8 else 0x7FFF) == zero).all()) for f in flat)


def test_table_zero_heads():
    """Per-head norm with a head of zeros, and a token of zeros: zeros out, like the oracle."""
    w = wl.TABLE_INTERLEAVED_T4096.with_(num_tokens=40)
    inputs = wl.table_inputs(w)
    inputs["q"] = inputs["q"].clone()
    inputs["k"] = inputs["k"].clone()
    inputs["q"][3, 5] = 0
    inputs["k"][9] = 0
    qo, ko = run_table(w, inputs)
    check_table_outputs(w.name, qo, ko, *oracle_table(w, inputs))
    assert bool((qo[3, 5].view(torch.int16) & 0x7FFF == 0).all())
    assert bool((ko[9].view(torch.int16) & 0x7FFF == 0).all())


# --- seeded sweep over the table contract -------------------------------------------------------

SWEEP_TABLE = [
    # (T, Hq, Hk, D, R, interleaved, norm_mode, table dtype)
    (7, 3, 1, 64, 64, True, "per_head", "f32"),
    (64, 2, 5, 128, 96, False, "per_head", "bf16"),
    (19, 4, 4, 96, 40, True, "per_head", "f32"),
    (33, 1, 2, 256, 256, True, "across_heads", "bf16"),
    (12, 3, 3, 32, 16, False, "across_heads", "f32"),
    (5, 2, 2, 8, 6, True, "none", "f32"),
    (9, 6, 2, 128, 128, False, "none", "bf16"),
    (1, 1, 1, 24, 2, True, "per_head", "bf16"),
    (40, 48, 8, 64, 32, True, "per_head", "f32"),
    (7, 5, 3, 256, 256, True, "per_head", "f32"),        # two tokens per workgroup, odd count
    (9, 10, 10, 128, 96, False, "across_heads", "bf16"),  # the same with across-heads norm
    # half-split with rotary_dim % 16 != 0: partners straddle 16-byte chunks
    (37, 3, 2, 64, 40, False, "per_head", "f32"),
    (50, 4, 4, 128, 100, False, "across_heads", "bf16"),
    (19, 2, 1, 32, 2, False, "none", "f32"),
    (23, 8, 8, 256, 250, False, "per_head", "bf16"),
    (11, 1, 3, 24, 8, False, "per_head", "f32"),
    (300, 24, 24, 128, 120, False, "per_head", "f32"),
]


@pytest.mark.parametrize("case", SWEEP_TABLE, ids=lambda c: "t{}_h{}-{}_d{}_r{}_{}_{}_{}".format(
    c[0], c[1], c[2], c[3], c[4], "il" if c[5] else "hs", c[6], c[7]))
def test_table_sweep(case):
    T, Hq, Hk, D, R, inter, mode, tdt = case
    w = wl.TableWorkload(name="sweep", num_tokens=T, num_heads_q=Hq, num_heads_k=Hk,
                         head_dim=D, rotary_dim=R, interleaved=inter, table_dtype=tdt,
                         seed=2000 + T + D, norm_mode=mode)
    inputs = wl.table_inputs(w)
    qo, ko = run_table(w, inputs)
    check_table_outputs(f"table {case}", qo, ko, *oracle_table(w, inputs))


def test_table_strided_views_and_in_place():
    """q and k as views into one packed [T, (Hq+Hk+pad)*D] buffer; outputs written in place."""
    T, Hq, Hk, D = 37, 3, 2, 64
    w = wl.TableWorkload(name="strided", num_tokens=T, num_heads_q=Hq, num_heads_k=Hk,
                         head_dim=D, rotary_dim=48, interleaved=True, table_dtype="f32", seed=77)
    inputs = wl.table_inputs(w)
    rq, rk = oracle_table(w, inputs)
    packed = torch.zeros(T, (Hq + Hk + 1) * D, dtype=torch.bfloat16, device=DEV)
    packed[:, :Hq * D] = _gpu(inputs["q"]).reshape(T, -1)
    packed[:, Hq * D:(Hq + Hk) * D] = _gpu(inputs["k"]).reshape(T, -1)
    tail = packed[:, (Hq + Hk) * D:].clone()
    q = packed[:, :Hq * D].view(T, Hq, D)
    k = packed[:, Hq * D:(Hq + Hk) * D].view(T, Hk, D)
    assert q.stride(0) == (Hq + Hk + 1) * D
    qr.qkrope_run_table(q, k, _gpu(inputs["q_weight"]), _gpu(inputs["k_weight"]),
                        _gpu(inputs["rope_table"]), w.eps, q_out=q, k_out=k, rotary_dim=48,
                        interleaved=True)
    torch.cuda.synchronize()
    check_table_outputs("in-place strided", q, k, rq, rk)
    assert torch.equal(packed[:, (Hq + Hk) * D:], tail)     # padding untouched


def test_table_page_signature():
    w = wl.TABLE_HALFSPLIT_T256.with_(num_tokens=20)
    inputs = wl.table_inputs(w)
    g = {n: _gpu(t) for n, t in inputs.items()}
    qo, ko = qr.fused_qk_norm_rope(g["q"], g["k"], g["q_weight"], g["k_weight"], g["rope_table"],
                                   w.eps, rotary_dim=w.rotary_dim, interleaved=False)
    torch.cuda.synchronize()
    check_table_outputs("page signature", qo, ko, *oracle_table(w, inputs))


# --- invariants between the two forms on the GPU ------------------------------------------------

@pytest.mark.parametrize("inter", [True, False])
@pytest.mark.parametrize("norm", [True, False])
def test_gpu_3d_equals_gpu_table_with_matching_table(inter, norm):
    """run_3d(x) == run_table(x's Q/K, table of the 3D angles), norm across heads or none."""
    w = wl.Rope3DWorkload(name="inv", batch=1, ppf=2, pph=3, ppw=5, num_frame_channels=16,
                          num_height_channels=24, num_width_channels=24, num_heads_q=4,
                          num_heads_k=2, num_heads_v=1, head_dim=64, seed=31, interleave=inter,
                          is_qk_norm=norm)
    inputs = wl.rope3d_inputs(w)
    q3, k3, _ = run_3d(w, inputs)
    D, T = w.head_dim, w.num_tokens
    f, h, ww = np.meshgrid(np.arange(w.ppf), np.arange(w.pph), np.arange(w.ppw), indexing="ij")
    pos = np.stack([f.ravel(), h.ravel(), ww.ravel()], 1)
    freqs = np.concatenate([w.base ** (-np.arange(0, c, 2) / c)
                            for c in (w.num_frame_channels, w.num_height_channels,
                                      w.num_width_channels)])
    axis = np.repeat([0, 1, 2], [w.num_frame_channels // 2, w.num_height_channels // 2,
                                 w.num_width_channels // 2])
    theta = pos[:, axis] * freqs
    tab = torch.from_numpy(np.ascontiguousarray(
        np.concatenate([np.cos(theta), np.sin(theta)], 1).astype(np.float32)))
    qkv = _gpu(inputs["qkv"]).reshape(T, -1)
    q = qkv[:, :w.num_heads_q * D].reshape(T, w.num_heads_q, D)
    k = qkv[:, w.num_heads_q * D:(w.num_heads_q + w.num_heads_k) * D].reshape(T, w.num_heads_k, D)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    qr.qkrope_run_table(q, k, _gpu(inputs["q_weight"]), _gpu(inputs["k_weight"]), _gpu(tab),
                        w.eps, q_out=qo, k_out=ko, interleaved=inter,
                        norm_mode="across_heads" if norm else "none")
    torch.cuda.synchronize()
    # both are bf16 roundings of values that agree to fp32 accuracy: at most one bf16 step apart
    assert_bf16_close(qo, q3.reshape(T, -1, D).double().cpu().numpy(), "q 3d vs table")
    assert_bf16_close(ko, k3.reshape(T, -1, D).double().cpu().numpy(), "k 3d vs table")


def test_gpu_position_zero_no_norm_is_identity():
    w = wl.Rope3DWorkload(name="id", batch=1, ppf=1, pph=1, ppw=1, num_frame_channels=64,
                          num_height_channels=32, num_width_channels=32, num_heads_q=3,
                          num_heads_k=3, num_heads_v=3, head_dim=128, seed=5, is_qk_norm=False)
    inputs = wl.rope3d_inputs(w)
    q, k, v = run_3d(w, inputs)
    qkv = _gpu(inputs["qkv"]).reshape(1, -1)
    assert torch.equal(q.reshape(1, -1), qkv[:, :3 * 128])
    assert torch.equal(k.reshape(1, -1), qkv[:, 3 * 128:6 * 128])
    assert torch.equal(v.reshape(1, -1), qkv[:, 6 * 128:])


# --- the boundary: validation and error mapping -------------------------------------------------

def test_empty_inputs_are_no_ops():
    w = wl.ROPE3D_ACROSS_S15360
    D = w.head_dim
    qkv = torch.empty(0, w.row_elems, dtype=torch.bfloat16, device=DEV)
    wq = torch.ones(w.num_heads_q * D, dtype=torch.bfloat16, device=DEV)
    q, k, v = qr.run_workload_3d(w, qkv, wq, wq)
    assert q.shape == (0, w.num_heads_q, D) and v.numel() == 0
    z = torch.empty(0, 2, 64, dtype=torch.bfloat16, device=DEV)
    tab = torch.empty(0, 64, dtype=torch.float32, device=DEV)
    w64 = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    qo, ko = qr.fused_qk_norm_rope(z, z, w64, w64, tab, 1e-6)
    assert qo.shape == z.shape


def test_contract_violations_raise_value_error():
    w = wl.ROPE3D_ACROSS_S15360.with_(ppf=1, pph=2, ppw=2)
    inputs = wl.rope3d_inputs(w)
    qkv, wq, wk = (_gpu(inputs[k]) for k in ("qkv", "q_weight", "k_weight"))
    base = dict(ppf=w.ppf, pph=w.pph, ppw=w.ppw, num_frame_channels=16, num_height_channels=56,
                num_width_channels=56, num_heads_q=32, num_heads_k=32, num_heads_v=32,
                head_dim=128)
    bad = [
        dict(num_frame_channels=18),                       # channels do not sum to head_dim
        dict(num_frame_channels=15, num_height_channels=57),  # odd channels
        dict(attention_factor=1.5),                        # attention factor without YaRN
        dict(factor=2.0, low=4.0, high=4.0),               # empty YaRN ramp
        dict(ppw=3),                                       # tokens not a multiple of seq_len
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            qr.fused_qk_rmsnorm_rope(qkv, wq, wk, **{**base, **kw})
    # head_dim outside {64, 128, 256} is rejected by the library itself
    x96 = torch.zeros(4, 3 * 96, dtype=torch.bfloat16, device=DEV)
    w96 = torch.ones(96, dtype=torch.bfloat16, device=DEV)
    o96 = [torch.empty(4, 1, 96, dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    with pytest.raises(ValueError, match="head_dim"):
        qr.qkrope_run_3d(x96, w96, w96, ppf=1, pph=2, ppw=2, num_frame_channels=32,
                         num_height_channels=32, num_width_channels=32, num_heads_q=1,
                         num_heads_k=1, num_heads_v=1, head_dim=96, q_out=o96[0], k_out=o96[1],
                         v_out=o96[2])
    # outputs overlapping the input are rejected by the library
    flat = qkv.view(-1, w.row_elems)
    q_alias = flat[:, :32 * 128].contiguous()
    with pytest.raises(ValueError):
        qr.qkrope_run_3d(flat, wq, wk, ppf=w.ppf, pph=w.pph, ppw=w.ppw, num_frame_channels=16,
                         num_height_channels=56, num_width_channels=56, num_heads_q=32,
                         num_heads_k=32, num_heads_v=32, head_dim=128,
                         q_out=flat.view(-1)[:q_alias.numel()].view(q_alias.shape),
                         k_out=torch.empty_like(q_alias), v_out=torch.empty_like(q_alias))
    # table-form head_dim above 256 is outside this library's kernels: unsupported
    t = wl.TableWorkload(name="u", num_tokens=4, num_heads_q=1, num_heads_k=1, head_dim=264,
                         rotary_dim=40, interleaved=False, table_dtype="f32", seed=3)
    ti = {n: _gpu(v) for n, v in wl.table_inputs(t).items()}
    with pytest.raises(ValueError, match="unsupported"):
        qr.fused_qk_norm_rope(ti["q"], ti["k"], ti["q_weight"], ti["k_weight"], ti["rope_table"],
                              1e-6, rotary_dim=40, interleaved=False)
    # norm weights shorter than what the kernels read are refused before any launch (the C ABI
    # takes bare pointers): [heads * head_dim] across heads, [head_dim] per head
    with pytest.raises(ValueError, match="q_weight"):
        qr.fused_qk_rmsnorm_rope(qkv, wq[:-8], wk, **base)
    with pytest.raises(ValueError, match="k_weight"):
        qr.fused_qk_rmsnorm_rope(qkv, wq, wk[:128], **base)
    t2 = t.with_(head_dim=64, rotary_dim=64, num_heads_q=2, num_heads_k=2)
    t2i = {n: _gpu(v) for n, v in wl.table_inputs(t2).items()}
    with pytest.raises(ValueError, match="k_weight"):
        qr.fused_qk_norm_rope(t2i["q"], t2i["k"], t2i["q_weight"], t2i["k_weight"][:32],
                              t2i["rope_table"], 1e-6)
    with pytest.raises(ValueError, match="q_weight"):
        qr.qkrope_run_table(t2i["q"], t2i["k"], t2i["q_weight"][:32], t2i["k_weight"],
                            t2i["rope_table"].float(), 1e-6, q_out=torch.empty_like(t2i["q"]),
                            k_out=torch.empty_like(t2i["k"]), norm_mode="across_heads")


def test_single_hip_runtime_loaded():
    qr.lib()
    runtimes = qr._hip_runtimes_loaded()
    assert len(runtimes) == 1, runtimes


@pytest.mark.parametrize("factor,base,inter,fp8", [
    (0.5, 10000.0, True, False),     # YaRN compressing positions the other way (factor < 1)
    (0.25, 3.0, False, True),        # and with a small base: angles of many turns
    (1.0, 0.5, True, False),         # base < 1: frequencies above one radian per position
    (3.0, 1.5, False, False),
], ids=lambda v: str(v))
def test_3d_yarn_factor_below_one_and_small_bases(factor, base, inter, fp8):
    """The contract takes any factor > 0 and base > 0; a factor below one raises the blended
    frequencies, and a small base gives angles of many turns (up to about 12 along the 40
    width positions), whose reduction to the period must hold to the usual tolerance at every
    position of a 6 x 7 x 40 grid."""
    yarn = factor != 1.0
    w = wl.Rope3DWorkload(name="yarn_edges", batch=2, ppf=6, pph=7, ppw=40,
                          num_frame_channels=32, num_height_channels=48, num_width_channels=48,
                          num_heads_q=6, num_heads_k=3, num_heads_v=2, head_dim=128,
                          seed=wl.SEED_BASE + 520, interleave=inter, base=base, factor=factor,
                          low=1.0 if yarn else 0.0, high=20.0 if yarn else 0.0,
                          attention_factor=0.9 if yarn else 1.0, output_fp8=fp8,
                          output_quant_scale=0.75 if fp8 else 1.0,
                          v_quant_scale=1.5 if fp8 else 1.0)
    inp = wl.rope3d_inputs(w)
    qkv, wq, wk = (inp[k].to(DEV) for k in ("qkv", "q_weight", "k_weight"))
    print(f"\nfactor {factor} base {base} interleave {inter} fp8 {fp8}", flush=True)
    outs = qr.run_workload_3d(w, qkv, wq, wk)
    torch.cuda.synchronize()
    ref = oracle.run_3d_workload(w, inp["qkv"].reshape(-1, w.row_elems), inp["q_weight"],
                                 inp["k_weight"])
    check_3d_outputs(w, outs, ref)
