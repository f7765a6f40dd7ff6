"""GPU parity for the extended contract, through the C ABI, against the fp64 oracle.

  * table form with IEEE binary16 activations (the table form's page: tables and outputs in
    "the activation dtype"), with float32 or binary16 tables;
  * separate [tokens, rotary_dim/2] cosine and sine tables (the SANA-WM camera prologue's
    rope_cos / rope_sin layout), with padded token strides;
  * E4M3 outputs for the table form;
  * grouped-query head counts (fewer K heads than Q heads);
  * the sharded 3D form: sequence shards with a global token offset (bit-identical to the
    unsharded launch), and head shards whose across-heads norm takes the per-token sums of
    squares reduced over every shard (qkrope_sumsq_3d, then qkrope_run_3d_sharded).
"""
from __future__ import annotations

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


def _gpu(t):
    return t.to(DEV)


def table_workload(T, Hq, Hk, D, R, inter, norm, act, tdt, seed, **kw):
    return wl.TableWorkload(name=f"ext_t{T}_h{Hq}-{Hk}_d{D}_r{R}", num_tokens=T, num_heads_q=Hq,
                            num_heads_k=Hk, head_dim=D, rotary_dim=R, interleaved=inter,
                            table_dtype=tdt, seed=seed, norm_mode=norm, act_dtype=act, **kw)


def oracle_table(w, inp, **kw):
    return oracle.run_table(inp["q"], inp["k"], inp["q_weight"], inp["k_weight"],
                            inp["rope_table"], w.eps, rotary_dim=w.rotary_dim,
                            interleaved=w.interleaved, norm_mode=w.norm_mode, **kw)


def split_views(tab, R, pad_c=8, pad_s=24):
    """Separate cos and sin GPU tables copied out of a packed [T, R] table, each inside a wider
    buffer so that its token stride is not R/2."""
    T = tab.shape[0]
    cbuf = torch.full((T, R // 2 + pad_c), 9.0, dtype=tab.dtype, device=DEV)
    sbuf = torch.full((T, R // 2 + pad_s), -9.0, dtype=tab.dtype, device=DEV)
    cbuf[:, : R // 2] = _gpu(tab[:, : R // 2])
    sbuf[:, : R // 2] = _gpu(tab[:, R // 2: R])
    return cbuf[:, : R // 2], sbuf[:, : R // 2]


# --- launches that write 2^27 bytes or more (stores at device scope through buffer resources) ---

def _run_table_full(w, inp):
    g = {k: _gpu(v) for k, v in inp.items()}
    odt = torch.float8_e4m3fn if w.out_dtype == "e4m3" else g["q"].dtype
    qo = torch.empty(g["q"].shape, dtype=odt, device=DEV)
    ko = torch.empty(g["k"].shape, dtype=odt, device=DEV)
    R = w.rotary_dim
    qr.qkrope_run_table_ex(g["q"], g["k"], g["q_weight"], g["k_weight"],
                           g["rope_table"][:, : R // 2], g["rope_table"][:, R // 2: R], w.eps,
                           q_out=qo, k_out=ko, rotary_dim=R, interleaved=w.interleaved,
                           norm_mode=w.norm_mode, out_scale=w.out_scale)
    torch.cuda.synchronize()
    return qo, ko


def _check_table(w, qo, ko, rq, rk):
    if w.out_dtype == "e4m3":
        assert_e4m3_within_one(qo, oracle.e4m3_encode(rq, w.out_scale), f"{w.name} q")
        assert_e4m3_within_one(ko, oracle.e4m3_encode(rk, w.out_scale), f"{w.name} k")
    elif w.act_dtype == "f16":
        assert_f16_close(qo, rq, f"{w.name} q")
        assert_f16_close(ko, rk, f"{w.name} k")
    else:
        assert_bf16_close(qo, rq, f"{w.name} q")
        assert_bf16_close(ko, rk, f"{w.name} k")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("w", [wl.TABLE_INTERLEAVED_T32768, wl.TABLE_INTERLEAVED_T32768_F16,
                               wl.TABLE_INTERLEAVED_T32768_E4M3], ids=lambda w: w.name)
def test_table_workload_full_size_every_token(w):
    """The 32768-token table workloads (403 MB, or 201 MB of E4M3 codes, written per launch:
    16- and 8-byte stores at device scope), every output element against the oracle."""
    inp = wl.table_inputs(w)
    qo, ko = _run_table_full(w, inp)
    _check_table(w, qo, ko, *oracle_table(w, inp))


@pytest.mark.parametrize("T", [32767, 32768])
def test_table_store_scope_threshold(T):
    """2 x 8 heads x 128 bf16 write 4096 bytes a token: 32767 tokens keep the global
    non-temporal stores, 32768 (2^27 bytes) store at device scope; both match the oracle."""
    w = table_workload(T, 8, 8, 128, 128, True, "per_head", "bf16", "bf16", seed=4700)
    inp = wl.table_inputs(w)
    qo, ko = _run_table_full(w, inp)
    _check_table(w, qo, ko, *oracle_table(w, inp))


# --- float16 activations -----------------------------------------------------------------------

F16_CASES = [
    # T, Hq, Hk, D, R, interleaved, norm mode, table dtype
    (333, 24, 24, 128, 128, True, "per_head", "f16"),
    (256, 4, 4, 128, 96, False, "per_head", "f32"),
    (97, 8, 2, 64, 32, False, "across_heads", "f16"),
    (64, 3, 5, 256, 200, True, "none", "f32"),
    (129, 6, 6, 128, 72, False, "per_head", "f16"),     # half-split, rotary_dim % 16 != 0
]


@pytest.mark.parametrize("case", F16_CASES, ids=lambda c: "t{}_h{}-{}_d{}_r{}_{}".format(*c[:5], c[7]))
def test_table_float16_activations(case):
    T, Hq, Hk, D, R, inter, norm, tdt = case
    w = table_workload(T, Hq, Hk, D, R, inter, norm, "f16", tdt, seed=4000 + T)
    inp = wl.table_inputs(w)
    g = {k: _gpu(v) for k, v in inp.items()}
    qo, ko = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    qr.qkrope_run_table_ex(g["q"], g["k"], g["q_weight"], g["k_weight"],
                           g["rope_table"][:, : R // 2], g["rope_table"][:, R // 2: R], w.eps,
                           q_out=qo, k_out=ko, rotary_dim=R, interleaved=inter, norm_mode=norm)
    torch.cuda.synchronize()
    rq, rk = oracle_table(w, inp)
    assert_f16_close(qo, rq, f"{w.name} q")
    assert_f16_close(ko, rk, f"{w.name} k")


def test_page_signature_accepts_float16():
    w = table_workload(200, 6, 6, 128, 96, False, "per_head", "f16", "f16", seed=4100)
    inp = wl.table_inputs(w)
    g = {k: _gpu(v) for k, v in inp.items()}
    qo, ko = qr.fused_qk_norm_rope(g["q"], g["k"], g["q_weight"], g["k_weight"], g["rope_table"],
                                   w.eps, rotary_dim=96, interleaved=False)
    torch.cuda.synchronize()
    rq, rk = oracle_table(w, inp)
    assert qo.dtype == torch.float16 and qo.shape == g["q"].shape
    assert_f16_close(qo, rq, "q")
    assert_f16_close(ko, rk, "k")


# --- separate cos / sin tables -----------------------------------------------------------------

@pytest.mark.parametrize("inter,R,tdt", [(True, 128, "bf16"), (False, 96, "f32"),
                                         (True, 62, "f32")])
def test_split_cos_sin_tables(inter, R, tdt):
    w = table_workload(515, 12, 4, 128, R, inter, "per_head", "bf16", tdt, seed=4200 + R)
    inp = wl.table_inputs(w)
    g = {k: _gpu(v) for k, v in inp.items()}
    cos_t, sin_t = split_views(inp["rope_table"], R)
    assert cos_t.stride(0) != sin_t.stride(0) != R // 2
    qo, ko = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    qr.qkrope_run_table_ex(g["q"], g["k"], g["q_weight"], g["k_weight"], cos_t, sin_t, w.eps,
                           q_out=qo, k_out=ko, rotary_dim=R, interleaved=inter)
    torch.cuda.synchronize()
    tab = inp["rope_table"]
    rq, rk = oracle.run_table(inp["q"], inp["k"], inp["q_weight"], inp["k_weight"],
                              tab[:, : R // 2].contiguous(), w.eps, rotary_dim=R,
                              interleaved=inter, sin_table=tab[:, R // 2: R].contiguous())
    assert_bf16_close(qo, rq, "q")
    assert_bf16_close(ko, rk, "k")
    # the packed-table entry point on the same inputs gives the same bits
    qp, kp = torch.empty_like(qo), torch.empty_like(ko)
    qr.qkrope_run_table(g["q"], g["k"], g["q_weight"], g["k_weight"], g["rope_table"], w.eps,
                        q_out=qp, k_out=kp, rotary_dim=R, interleaved=inter)
    torch.cuda.synchronize()
    assert torch.equal(qp, qo) and torch.equal(kp, ko)


# --- E4M3 outputs for the table form -----------------------------------------------------------

@pytest.mark.parametrize("act,inter,scale,sigma,R", [("bf16", True, 0.5, 1.0, 128),
                                                     ("f16", False, 2.0, 1.0, 96),
                                                     ("bf16", False, 300.0, 4.0, 96),
                                                     ("bf16", False, 1.0, 1.0, 52)])
def test_table_e4m3_outputs(act, inter, scale, sigma, R):
    w = table_workload(301, 16, 8, 128, R, inter, "per_head", act, "f32",
                       seed=4300 + int(scale) + R, sigma=sigma)
    inp = wl.table_inputs(w)
    g = {k: _gpu(v) for k, v in inp.items()}
    R = w.rotary_dim
    qo = torch.empty(g["q"].shape, dtype=torch.float8_e4m3fn, device=DEV)
    ko = torch.empty(g["k"].shape, dtype=torch.float8_e4m3fn, device=DEV)
    qr.qkrope_run_table_ex(g["q"], g["k"], g["q_weight"], g["k_weight"],
                           g["rope_table"][:, : R // 2], g["rope_table"][:, R // 2: R], w.eps,
                           q_out=qo, k_out=ko, rotary_dim=R, interleaved=inter, out_scale=scale)
    torch.cuda.synchronize()
    rq, rk = oracle_table(w, inp)
    assert_e4m3_within_one(qo, oracle.e4m3_encode(rq, scale), "q")
    assert_e4m3_within_one(ko, oracle.e4m3_encode(rk, scale), "k")
    if scale >= 300:
        codes = qo.view(torch.uint8).cpu().numpy()
        assert ((codes & 0x7F) == 0x7E).any(), "the saturation case must reach +-448"


# E4M3 outputs at head_dim == rotary_dim == 128 with one slot per region run a kernel whose head
# geometry is fixed at compile time: every norm, both pairings, both table formats, one token per
# workgroup (3, 16 or 24 Q heads) and two (2 or 6 heads per region fill 32 + 64k lanes),
# saturation.
@pytest.mark.parametrize("inter,norm,act,tdt,hq,hk,scale,sigma", [
    (True, "per_head", "bf16", "f32", 16, 8, 0.5, 1.0),
    (False, "across_heads", "bf16", "bf16", 6, 6, 1.0, 1.0),
    (True, "none", "bf16", "bf16", 2, 2, 1.0, 1.0),
    (False, "per_head", "f16", "f32", 2, 2, 2.0, 1.0),
    (True, "across_heads", "f16", "f16", 24, 24, 1.0, 1.0),
    (False, "none", "bf16", "f32", 3, 3, 300.0, 4.0),
])
def test_table_e4m3_head_dim_128(inter, norm, act, tdt, hq, hk, scale, sigma):
    w = table_workload(301, hq, hk, 128, 128, inter, norm, act, tdt, seed=4350 + hq + hk,
                       sigma=sigma)
    w = w.with_(out_dtype="e4m3", out_scale=scale)
    inp = wl.table_inputs(w)
    g = {k: _gpu(v) for k, v in inp.items()}
    qo = torch.empty(g["q"].shape, dtype=torch.float8_e4m3fn, device=DEV)
    ko = torch.empty(g["k"].shape, dtype=torch.float8_e4m3fn, device=DEV)
    qr.qkrope_run_table_ex(g["q"], g["k"], g["q_weight"], g["k_weight"],
                           g["rope_table"][:, :64], g["rope_table"][:, 64:], w.eps,
                           q_out=qo, k_out=ko, rotary_dim=128, interleaved=inter,
                           norm_mode=norm, out_scale=scale)
    torch.cuda.synchronize()
    rq, rk = oracle_table(w, inp)
    assert_e4m3_within_one(qo, oracle.e4m3_encode(rq, scale), "q")
    assert_e4m3_within_one(ko, oracle.e4m3_encode(rk, scale), "k")
    if scale >= 300:
        codes = qo.view(torch.uint8).cpu().numpy()
        assert ((codes & 0x7F) == 0x7E).any(), "the saturation case must reach +-448"


def test_table_ex_contract():
    w = table_workload(16, 2, 2, 64, 64, True, "per_head", "f16", "f16", seed=4400)
    inp = wl.table_inputs(w)
    g = {k: _gpu(v) for k, v in inp.items()}
    c, s = g["rope_table"][:, :32], g["rope_table"][:, 32:]
    qo, ko = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    with pytest.raises(ValueError):         # bf16 table with float16 activations
        qr.qkrope_run_table_ex(g["q"], g["k"], g["q_weight"], g["k_weight"], c.bfloat16(),
                               s.bfloat16(), 1e-6, q_out=qo, k_out=ko)
    with pytest.raises(ValueError):         # bf16 outputs for float16 activations
        qr.qkrope_run_table_ex(g["q"], g["k"], g["q_weight"], g["k_weight"], c, s, 1e-6,
                               q_out=qo.bfloat16(), k_out=ko.bfloat16())
    q8 = g["q"].view(torch.float8_e4m3fn)[..., :64].contiguous()
    with pytest.raises(ValueError):         # E4M3 needs a positive finite scale
        qr.qkrope_run_table_ex(g["q"], g["k"], g["q_weight"], g["k_weight"], c, s, 1e-6,
                               q_out=q8, k_out=torch.empty_like(q8), out_scale=0.0)
    # E4M3 output written over its own 16-bit input is rejected (different element size)
    L = qr.lib()
    rc = L.qkrope_run_table_ex(qr._handle_for(g["q"].device), g["q"].data_ptr(),
                               g["k"].data_ptr(), g["q_weight"].data_ptr(),
                               g["k_weight"].data_ptr(), c.data_ptr(), s.data_ptr(),
                               qr.QKROPE_DTYPE_F16, qr.QKROPE_DTYPE_F16, qr.QKROPE_DTYPE_E4M3,
                               1.0, 1e-6, 16, 2, 2, 64, 64, 1, 1, 128, 128, 64, 64,
                               g["q"].data_ptr(), ko.data_ptr(), 128, 128, None)
    assert rc == qr.QKROPE_ERR_INVALID
    # token strides of 2^28 elements or more are refused (rows are addressed with 32-bit
    # byte offsets inside a workgroup); one token keeps every span inside the buffers
    for qs, qos in ((1 << 28, 128), (128, 1 << 28)):
        rc = L.qkrope_run_table_ex(qr._handle_for(g["q"].device), g["q"].data_ptr(),
                                   g["k"].data_ptr(), g["q_weight"].data_ptr(),
                                   g["k_weight"].data_ptr(), c.data_ptr(), s.data_ptr(),
                                   qr.QKROPE_DTYPE_F16, qr.QKROPE_DTYPE_F16, qr.QKROPE_DTYPE_F16,
                                   1.0, 1e-6, 1, 2, 2, 64, 64, 1, 1, qs, 128, 64, 64,
                                   qo.data_ptr(), ko.data_ptr(), qos, 128, None)
        assert rc == qr.QKROPE_ERR_UNSUPPORTED


# --- grouped-query head counts -----------------------------------------------------------------

@pytest.mark.parametrize("inter", [True, False])
def test_table_gqa(inter):
    w = table_workload(700, 32, 4, 128, 128, inter, "per_head", "bf16", "bf16", seed=4500)
    inp = wl.table_inputs(w)
    g = {k: _gpu(v) for k, v in inp.items()}
    qo, ko = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    qr.qkrope_run_table(g["q"], g["k"], g["q_weight"], g["k_weight"], g["rope_table"], w.eps,
                        q_out=qo, k_out=ko, rotary_dim=128, interleaved=inter)
    torch.cuda.synchronize()
    rq, rk = oracle_table(w, inp)
    assert_bf16_close(qo, rq, "q")
    assert_bf16_close(ko, rk, "k")


@pytest.mark.parametrize("inter,fp8", [(True, False), (False, True)])
def test_3d_gqa(inter, fp8):
    w = wl.Rope3DWorkload(name="gqa3d", batch=1, ppf=3, pph=8, ppw=10, num_frame_channels=16,
                          num_height_channels=56, num_width_channels=56, num_heads_q=24,
                          num_heads_k=4, num_heads_v=4, head_dim=128, seed=4600,
                          interleave=inter, output_fp8=fp8, output_quant_scale=0.5,
                          v_quant_scale=0.25)
    inp = wl.rope3d_inputs(w)
    outs = qr.run_workload_3d(w, *(_gpu(inp[k]) for k in ("qkv", "q_weight", "k_weight")))
    torch.cuda.synchronize()
    ref = oracle.run_3d_workload(w, inp["qkv"].reshape(-1, w.row_elems), inp["q_weight"],
                                 inp["k_weight"])
    check_3d_outputs(w, outs, ref)


# --- the sharded 3D form -----------------------------------------------------------------------

def _kw(w):
    return dict(ppf=w.ppf, pph=w.pph, ppw=w.ppw, num_frame_channels=w.num_frame_channels,
                num_height_channels=w.num_height_channels, num_width_channels=w.num_width_channels,
                head_dim=w.head_dim, eps=w.eps, base=w.base, interleave=w.interleave,
                factor=w.factor, low=w.low, high=w.high, attention_factor=w.attention_factor,
                is_qk_norm=w.is_qk_norm, output_fp8=w.output_fp8,
                output_quant_scale=w.output_quant_scale, v_quant_scale=w.v_quant_scale)


def _outs(T, w, Hq, Hk, Hv):
    odt = torch.float8_e4m3fn if w.output_fp8 else torch.bfloat16
    return [torch.empty((T, H, w.head_dim), dtype=odt, device=DEV) for H in (Hq, Hk, Hv)]


@pytest.mark.parametrize("w", [wl.ROPE3D_ACROSS_S15360.with_(ppf=2),
                               wl.ROPE3D_NEOX_FP8_S18480.with_(ppf=2, pph=7),
                               wl.ROPE3D_YARN_S122880.with_(ppf=1, pph=9)],
                         ids=lambda w: w.name)
def test_sequence_shards_match_unsharded_bits(w):
    inp = wl.rope3d_inputs(w)
    qkv, wq, wk = (_gpu(inp[k]) for k in ("qkv", "q_weight", "k_weight"))
    full = qr.run_workload_3d(w, qkv, wq, wk)
    x = qkv.reshape(-1, w.row_elems)
    T = w.num_tokens
    cuts = [0, 7, T // 3, T // 2 + 5, T - 1, T]        # uneven, crossing sequence boundaries
    parts = [[], [], []]
    for a, b in zip(cuts[:-1], cuts[1:]):
        outs = _outs(b - a, w, w.num_heads_q, w.num_heads_k, w.num_heads_v)
        qr.qkrope_run_3d_sharded(x[a:b].contiguous(), wq, wk, token_offset=a,
                                 num_heads_q=w.num_heads_q, num_heads_k=w.num_heads_k,
                                 num_heads_v=w.num_heads_v, q_out=outs[0], k_out=outs[1],
                                 v_out=outs[2], **_kw(w))
        for i in range(3):
            parts[i].append(outs[i])
    torch.cuda.synchronize()
    for i in range(3):
        got = torch.cat(parts[i]).view(torch.uint8)
        assert torch.equal(got, full[i].reshape(got.shape[0], -1, w.head_dim).view(torch.uint8)), \
            f"region {'qkv'[i]} differs from the unsharded launch"


@pytest.mark.parametrize("w,tp", [(wl.ROPE3D_ACROSS_S15360.with_(ppf=2), 4),
                                  (wl.ROPE3D_NEOX_FP8_S18480.with_(ppf=2, pph=7), 5)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_head_shards_two_phase_norm(w, tp):
    inp = wl.rope3d_inputs(w)
    T, D = w.num_tokens, w.head_dim
    Hq, Hk, Hv = w.num_heads_q, w.num_heads_k, w.num_heads_v
    assert Hq % tp == 0 and Hk % tp == 0 and Hv % tp == 0
    x = _gpu(inp["qkv"]).reshape(T, Hq + Hk + Hv, D)
    wq, wk = _gpu(inp["q_weight"]), _gpu(inp["k_weight"])
    hq, hk, hv = Hq // tp, Hk // tp, Hv // tp
    shards = []
    for r in range(tp):
        sq, sk, sv = slice(r * hq, (r + 1) * hq), slice(Hq + r * hk, Hq + (r + 1) * hk), \
            slice(Hq + Hk + r * hv, Hq + Hk + (r + 1) * hv)
        shards.append(torch.cat([x[:, sq], x[:, sk], x[:, sv]], dim=1).reshape(T, -1).contiguous())
    # phase 1 on every rank, then the sum over ranks (the all-reduce of a head group)
    partial = [qr.qkrope_sumsq_3d(s, num_heads_q=hq, num_heads_k=hk, num_heads_v=hv, head_dim=D)
               for s in shards]
    total = torch.stack(partial).sum(dim=0)
    torch.cuda.synchronize()
    ref_total = oracle.sumsq_3d(inp["qkv"].reshape(T, -1), num_heads_q=Hq, num_heads_k=Hk,
                                num_heads_v=Hv, head_dim=D)
    np.testing.assert_allclose(total.cpu().numpy(), ref_total, rtol=1e-5)
    ref0 = oracle.sumsq_3d(shards[0].cpu(), num_heads_q=hq, num_heads_k=hk, num_heads_v=hv,
                           head_dim=D)
    np.testing.assert_allclose(partial[0].cpu().numpy(), ref0, rtol=1e-5)
    # phase 2 on every rank, outputs gathered back along heads
    outs = []
    for r, s in enumerate(shards):
        o = _outs(T, w, hq, hk, hv)
        qr.qkrope_run_3d_sharded(s, wq[r * hq * D:(r + 1) * hq * D],
                                 wk[r * hk * D:(r + 1) * hk * D], sumsq=total,
                                 norm_elems_q=Hq * D, norm_elems_k=Hk * D, num_heads_q=hq,
                                 num_heads_k=hk, num_heads_v=hv, q_out=o[0], k_out=o[1],
                                 v_out=o[2], **_kw(w))
        outs.append(o)
    torch.cuda.synchronize()
    gathered = [torch.cat([o[i] for o in outs], dim=1) for i in range(3)]
    ref = oracle.run_3d_workload(w, inp["qkv"].reshape(T, -1), inp["q_weight"], inp["k_weight"])
    check_3d_outputs(w, gathered, ref)


def test_sharded_contract():
    w = wl.ROPE3D_ACROSS_S15360.with_(ppf=1, pph=2, ppw=4, batch=1)
    inp = wl.rope3d_inputs(w)
    qkv, wq, wk = (_gpu(inp[k]) for k in ("qkv", "q_weight", "k_weight"))
    T = w.num_tokens
    o = _outs(T, w, w.num_heads_q, w.num_heads_k, w.num_heads_v)
    base = dict(num_heads_q=w.num_heads_q, num_heads_k=w.num_heads_k, num_heads_v=w.num_heads_v,
                q_out=o[0], k_out=o[1], v_out=o[2], **_kw(w))
    with pytest.raises(ValueError, match="token_offset"):
        qr.qkrope_run_3d_sharded(qkv, wq, wk, token_offset=-1, **base)
    with pytest.raises(ValueError, match="2\\^31"):
        qr.qkrope_run_3d_sharded(qkv, wq, wk, token_offset=(1 << 31) - 4, **base)
    s = torch.ones((T, 2), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError, match="norm_elems"):
        qr.qkrope_run_3d_sharded(qkv, wq, wk, sumsq=s, norm_elems_q=8, norm_elems_k=8, **base)
    # a shard need not hold whole sequences
    o5 = _outs(5, w, w.num_heads_q, w.num_heads_k, w.num_heads_v)
    qr.qkrope_run_3d_sharded(qkv.reshape(T, -1)[:5].contiguous(), wq, wk, token_offset=3,
                             **{**base, "q_out": o5[0], "k_out": o5[1], "v_out": o5[2]})
    torch.cuda.synchronize()
    ref = oracle.run_3d_workload(w, inp["qkv"].reshape(T, -1)[:5], inp["q_weight"],
                                 inp["k_weight"], token_offset=3)
    assert_bf16_close(o5[0], ref[0], "q of a 5-token shard at offset 3")


@pytest.mark.parametrize("fp8", [False, True])
def test_sharded_largest_token_offset(fp8):
    """Positions come from (token_offset + t) split by the grid with magic divisors that hold
    for indices below 2^31: a shard ending at global index 2^31 - 1, on a 3 x 5 x 7 grid."""
    w = wl.Rope3DWorkload(name="offset_top", batch=1, ppf=3, pph=5, ppw=7,
                          num_frame_channels=16, num_height_channels=24, num_width_channels=24,
                          num_heads_q=3, num_heads_k=2, num_heads_v=1, head_dim=64,
                          seed=wl.SEED_BASE + 530, output_fp8=fp8,
                          output_quant_scale=0.5 if fp8 else 1.0,
                          v_quant_scale=2.0 if fp8 else 1.0)
    inp = wl.rope3d_inputs(w)
    qkv, wq, wk = (_gpu(inp[k]) for k in ("qkv", "q_weight", "k_weight"))
    T = w.num_tokens
    off = (1 << 31) - 1 - T
    o = _outs(T, w, w.num_heads_q, w.num_heads_k, w.num_heads_v)
    qr.qkrope_run_3d_sharded(qkv.reshape(T, -1), wq, wk, token_offset=off,
                             num_heads_q=w.num_heads_q, num_heads_k=w.num_heads_k,
                             num_heads_v=w.num_heads_v, q_out=o[0], k_out=o[1], v_out=o[2],
                             **_kw(w))
    torch.cuda.synchronize()
    ref = oracle.run_3d_workload(w, inp["qkv"].reshape(T, -1), inp["q_weight"],
                                 inp["k_weight"], token_offset=off)
    check_3d_outputs(w, o, ref)


# --- regions without heads (their tensors may be empty, with NULL data pointers) ----------------

@pytest.mark.parametrize("none_weight", [False, True], ids=["empty_weight", "none_weight"])
@pytest.mark.parametrize("hq,hk,inter,mode", [(0, 27, True, "across_heads"), (5, 0, False, "across_heads"),
                                              (0, 9, False, "per_head"), (12, 0, True, "none")])
def test_table_empty_region_null_pointers(hq, hk, inter, mode, none_weight):
    w = table_workload(153, hq, hk, 200, 146 if inter else 96, inter, mode, "bf16", "bf16",
                       seed=4700 + hq + hk)
    inp = wl.table_inputs(w)
    g = {k: _gpu(v) for k, v in inp.items()}
    assert (g["q"].data_ptr() == 0) == (hq == 0) and (g["k"].data_ptr() == 0) == (hk == 0)
    if none_weight:         # the weight of a region without heads may also be None
        g["q_weight"] = g["q_weight"] if hq else None
        g["k_weight"] = g["k_weight"] if hk else None
    qo, ko = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    R = w.rotary_dim
    qr.qkrope_run_table_ex(g["q"], g["k"], g["q_weight"], g["k_weight"],
                           g["rope_table"][:, : R // 2], g["rope_table"][:, R // 2: R], w.eps,
                           q_out=qo, k_out=ko, rotary_dim=R, interleaved=inter, norm_mode=mode)
    torch.cuda.synchronize()
    rq, rk = oracle_table(w, inp)
    if hq:
        assert_bf16_close(qo, rq, "q")
    if hk:
        assert_bf16_close(ko, rk, "k")


@pytest.mark.parametrize("none_weight", [False, True], ids=["empty_weight", "none_weight"])
@pytest.mark.parametrize("H,norm", [((0, 0, 6), True), ((4, 0, 0), True), ((0, 3, 0), True),
                                    ((0, 5, 2), True)])
def test_3d_empty_regions_null_weights(H, norm, none_weight):
    w = wl.Rope3DWorkload(name="empty3d", batch=2, ppf=2, pph=3, ppw=5, num_frame_channels=32,
                          num_height_channels=48, num_width_channels=48, num_heads_q=H[0],
                          num_heads_k=H[1], num_heads_v=H[2], head_dim=128, seed=4800 + sum(H),
                          is_qk_norm=norm)
    inp = wl.rope3d_inputs(w)
    qkv, wq, wk = (_gpu(inp[k]) for k in ("qkv", "q_weight", "k_weight"))
    assert (wq.data_ptr() == 0) == (H[0] == 0) and (wk.data_ptr() == 0) == (H[1] == 0)
    if none_weight:
        wq, wk = (wq if H[0] else None), (wk if H[1] else None)
    outs = qr.run_workload_3d(w, qkv, wq, wk)
    torch.cuda.synchronize()
    ref = oracle.run_3d_workload(w, inp["qkv"].reshape(-1, w.row_elems), inp["q_weight"],
                                 inp["k_weight"])
    check_3d_outputs(w, outs, ref)
    s = qr.qkrope_sumsq_3d(qkv, num_heads_q=H[0], num_heads_k=H[1], num_heads_v=H[2],
                           head_dim=128)
    torch.cuda.synchronize()
    ref_s = oracle.sumsq_3d(inp["qkv"].reshape(w.num_tokens, -1), num_heads_q=H[0],
                            num_heads_k=H[1], num_heads_v=H[2], head_dim=128)
    np.testing.assert_allclose(s.cpu().numpy(), ref_s, rtol=1e-5)


# --- streams and graphs --------------------------------------------------------------------------

def test_concurrent_streams_one_handle():
    # the handle is immutable: calls on two streams at once give the single-stream results
    ws = [wl.ROPE3D_ACROSS_S15360.with_(ppf=1, pph=4), wl.ROPE3D_NEOX_FP8_S18480.with_(ppf=1, pph=5)]
    ins = [wl.rope3d_inputs(w) for w in ws]
    g = [{k: _gpu(v) for k, v in i.items()} for i in ins]
    ref = [qr.run_workload_3d(w, x["qkv"], x["q_weight"], x["k_weight"]) for w, x in zip(ws, g)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty_like(o) for o in r] for r in ref]
    for rep in range(5):
        for w, x, o, st in zip(ws, g, outs, streams):
            with torch.cuda.stream(st):
                qr.run_workload_3d(w, x["qkv"], x["q_weight"], x["k_weight"], *o)
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            for a, b in zip(o, r):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_graph_capture_and_replay():
    # both forms captured in one HIP graph; every replay matches the eager launch bit for bit
    w3 = wl.ROPE3D_ACROSS_S15360.with_(ppf=1, pph=6)
    wt = wl.TABLE_INTERLEAVED_T4096.with_(num_tokens=777)
    i3 = {k: _gpu(v) for k, v in wl.rope3d_inputs(w3).items()}
    it = {k: _gpu(v) for k, v in wl.table_inputs(wt).items()}
    o3 = qr.run_workload_3d(w3, i3["qkv"], i3["q_weight"], i3["k_weight"])
    qo, ko = torch.empty_like(it["q"]), torch.empty_like(it["k"])
    eager = lambda: (qr.run_workload_3d(w3, i3["qkv"], i3["q_weight"], i3["k_weight"], *o3),
                     qr.qkrope_run_table(it["q"], it["k"], it["q_weight"], it["k_weight"],
                                         it["rope_table"], wt.eps, q_out=qo, k_out=ko,
                                         interleaved=True))
    eager()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (*o3, qo, ko)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        eager()                                   # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            eager()
    for rep in range(4):
        for t in (*o3, qo, ko):
            t.zero_()                             # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip((*o3, qo, ko), ref):
            assert torch.equal(t, r), f"replay {rep}"


def test_graph_replay_sharded_step_and_e4m3_outputs():
    """The two-kernel sharded step (sums of squares, then the apply that reads them), the FP8
    3D form and the split-table form with E4M3 outputs, captured in one HIP graph: every replay,
    with the outputs and the sums cleared eagerly in between, matches the eager launch bit for
    bit."""
    ws = wl.ROPE3D_ACROSS_S15360_TP4.with_(ppf=1, pph=4)
    w8 = wl.ROPE3D_NEOX_FP8_S18480.with_(ppf=1, pph=4)
    wt = table_workload(333, 6, 2, 128, 128, False, "per_head", "bf16", "f32", seed=4900,
                        out_dtype="e4m3", out_scale=0.8)
    i_s = {k: _gpu(v) for k, v in wl.rope3d_inputs(ws).items()}
    i8 = {k: _gpu(v) for k, v in wl.rope3d_inputs(w8).items()}
    it = {k: _gpu(v) for k, v in wl.table_inputs(wt).items()}
    Ts = ws.num_tokens
    so = _outs(Ts, ws, ws.num_heads_q, ws.num_heads_k, ws.num_heads_v)
    sums = torch.empty((Ts, 2), dtype=torch.float32, device=DEV)
    o8 = qr.run_workload_3d(w8, i8["qkv"], i8["q_weight"], i8["k_weight"])
    f8 = torch.float8_e4m3fn
    qo = torch.empty(it["q"].shape, dtype=f8, device=DEV)
    ko = torch.empty(it["k"].shape, dtype=f8, device=DEV)
    R = wt.rotary_dim
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):      # the prepared step keeps the stream current at its creation
        prep = qr.PreparedSharded3D(ws, i_s["qkv"], i_s["q_weight"], i_s["k_weight"], *so, sums,
                                    sums)

    def eager():
        prep()
        qr.run_workload_3d(w8, i8["qkv"], i8["q_weight"], i8["k_weight"], *o8)
        qr.qkrope_run_table_ex(it["q"], it["k"], it["q_weight"], it["k_weight"],
                               it["rope_table"][:, : R // 2], it["rope_table"][:, R // 2: R],
                               wt.eps, q_out=qo, k_out=ko, rotary_dim=R, interleaved=False,
                               out_scale=wt.out_scale)

    outs = (*so, sums, *o8, qo, ko)
    with torch.cuda.stream(s):
        eager()
    torch.cuda.synchronize()
    ref = [t.view(torch.uint8).clone() if t.dtype == f8 else t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            eager()
    for rep in range(4):
        for t in outs:
            (t.view(torch.uint8) if t.dtype == f8 else t).zero_()    # eager work between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            got = t.view(torch.uint8) if t.dtype == f8 else t
            assert torch.equal(got, r), f"replay {rep}"


@pytest.mark.timeout(600)
def test_graph_replay_full_size_named_3d_workloads():
    """The three large 3D workloads at full size, launched as bench.py times them: marshalled
    once (Prepared3D, on the capture stream) and replayed from one HIP graph. Every output is
    stored at device scope there (each launch writes 142 MB to 3 GB). Every replay, with the
    outputs cleared eagerly in between, matches the eager launch bit for bit; the eager launch
    itself matches the oracle at every token (tests/test_gpu_parity.py)."""
    ws = [wl.ROPE3D_ACROSS_S15360, wl.ROPE3D_NEOX_FP8_S18480, wl.ROPE3D_YARN_S122880]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    preps, outs = [], []
    with torch.cuda.stream(s):
        for w in ws:
            x = {k: _gpu(v) for k, v in wl.rope3d_inputs(w).items()}
            o = qr.run_workload_3d(w, x["qkv"], x["q_weight"], x["k_weight"])
            preps.append(qr.Prepared3D(w, x["qkv"], x["q_weight"], x["k_weight"], *o))
            outs.extend(o)
    torch.cuda.synchronize()
    raw = [t.view(torch.uint8) for t in outs]
    ref = [t.clone() for t in raw]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for prep in preps:
                prep()
    for rep in range(3):
        for t in raw:
            t.zero_()                             # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for w, t, r in zip([w for w in ws for _ in range(3)], raw, ref):
            assert torch.equal(t, r), f"{w.name}, replay {rep}"


@pytest.mark.timeout(600)
def test_graph_replay_full_size_tables_and_camera():
    """The 32768-token table workloads and the three camera-prologue workloads at full size,
    marshalled once (PreparedTable, PreparedCam) and replayed from one HIP graph, as bench.py
    times them: every replay, with the outputs cleared eagerly in between, matches the eager
    launch bit for bit (whose outputs match the oracle at every element elsewhere)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    preps, outs, names = [], [], []
    with torch.cuda.stream(s):
        for w in (wl.TABLE_INTERLEAVED_T32768, wl.TABLE_INTERLEAVED_T32768_F16,
                  wl.TABLE_INTERLEAVED_T32768_E4M3):
            g = {k: _gpu(v) for k, v in wl.table_inputs(w).items()}
            odt = torch.float8_e4m3fn if w.out_dtype == "e4m3" else g["q"].dtype
            qo = torch.empty(g["q"].shape, dtype=odt, device=DEV)
            ko = torch.empty(g["k"].shape, dtype=odt, device=DEV)
            preps.append(qr.PreparedTable(g["q"], g["k"], g["q_weight"], g["k_weight"],
                                          g["rope_table"], w.eps, q_out=qo, k_out=ko,
                                          rotary_dim=w.rotary_dim, interleaved=w.interleaved,
                                          norm_mode=w.norm_mode, out_scale=w.out_scale))
            outs += [qo, ko]
            names += [w.name] * 2
        for w in (wl.CAM_PREP_S18480, wl.CAM_PREP_S18432, wl.CAM_PREP_S18480_P18496):
            g = {k: _gpu(v) for k, v in wl.cam_inputs(w).items()}
            B, N, H, D = w.batch, w.num_tokens, w.num_heads, w.head_dim
            o = [torch.empty((B, H, D, w.out_pitch), dtype=g["q"].dtype, device=DEV)[..., :N]
                 for _ in range(3)]
            infl = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
            preps.append(qr.PreparedCam(g["q"], g["k"], g["v"], g["proj_q"], g["proj_kv"],
                                        g["rope_cos"], g["rope_sin"], w.k_scale, *o, infl))
            outs += [*o, infl]
            names += [w.name] * 4
    torch.cuda.synchronize()
    raw = [t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t for t in outs]
    ref = [t.clone() for t in raw]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for prep in preps:
                prep()
    for rep in range(3):
        for t in raw:
            t.zero_()                             # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(names, raw, ref):
            assert torch.equal(t, r), f"{name}, replay {rep}"


def test_host_tensor_arguments_are_refused():
    """A host tensor among GPU ones (weights, tables, outputs, matrices) raises before launch."""
    wt = wl.TABLE_INTERLEAVED_T4096.with_(num_tokens=64)
    ti = wl.table_inputs(wt)
    g = {k: _gpu(v) for k, v in ti.items()}
    qo, ko = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    with pytest.raises(ValueError, match="GPU"):
        qr.qkrope_run_table(g["q"], g["k"], ti["q_weight"], g["k_weight"], g["rope_table"],
                            wt.eps, q_out=qo, k_out=ko, interleaved=True)
    with pytest.raises(ValueError, match="GPU"):
        qr.qkrope_run_table(g["q"], g["k"], g["q_weight"], g["k_weight"], g["rope_table"],
                            wt.eps, q_out=qo, k_out=ko.cpu(), interleaved=True)
    w3 = wl.ROPE3D_ACROSS_S15360.with_(ppf=1, pph=1, ppw=8)
    i3 = wl.rope3d_inputs(w3)
    outs = [torch.empty((w3.num_tokens, 32, 128), dtype=torch.bfloat16, device=DEV)
            for _ in range(3)]
    with pytest.raises(ValueError, match="GPU"):
        qr.qkrope_run_3d(_gpu(i3["qkv"]), i3["q_weight"], _gpu(i3["k_weight"]), ppf=1, pph=1,
                         ppw=8, num_frame_channels=16, num_height_channels=56,
                         num_width_channels=56, num_heads_q=32, num_heads_k=32, num_heads_v=32,
                         head_dim=128, q_out=outs[0], k_out=outs[1], v_out=outs[2])
    wc = wl.CAM_PREP_S18480.with_(batch=1, ppf=1, pph=1, ppw=16, num_heads=2)
    ci = wl.cam_inputs(wc)
    gc = {k: _gpu(v) for k, v in ci.items()}
    co = [torch.empty((1, 2, 64, 16), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    with pytest.raises(ValueError, match="GPU"):
        qr.qkrope_cam_prep(gc["q"], gc["k"], gc["v"], ci["proj_q"], gc["proj_kv"],
                           gc["rope_cos"], gc["rope_sin"], 1.0, q_out=co[0], k_out=co[1],
                           v_out=co[2])
    torch.cuda.synchronize()
