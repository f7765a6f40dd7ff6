"""GPU parity of the camera prologue (qkrope_cam_prep; vLLM-Omni "vllm_omni.diffusion.models.
sana_wm.ucpe", cam_prep_func) against the fp64 oracle, through the C ABI.

Shapes cover several 64-token tiles with a ragged tail, token counts that are and are not
multiples of 8 (16-byte and element stores), one and two chunks per lane, chunk counts that
do not fill a power-of-two lane group, uneven head groups, a single token, binary16, padded
token strides, padded output rows, no inflation output, empty problems, argument errors, graph
replay, and the full-size SANA-WM shapes at every token.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from parity import assert_cam_close, assert_inflation_close, to_f64

pytestmark = pytest.mark.gpu

qr = pytest.importorskip("qk_rmsnorm_rope_amd")
from qk_rmsnorm_rope_amd import workloads as wl  # noqa: E402

DEV = "cuda"


def workload(B, N, H, D, act="bf16", seed=0):
    return wl.CamWorkload(name=f"cam_b{B}_n{N}_h{H}_d{D}_{act}", batch=B, ppf=1, pph=1, ppw=N,
                          num_heads=H, head_dim=D, seed=wl.SEED_BASE + 500 + seed, act_dtype=act)


def gpu_inputs(inp):
    return {k: v.to(DEV) for k, v in inp.items()}


PAD_BITS = 0x7FA5       # a NaN pattern in both 16-bit formats, written into output padding


def run_gpu(g, k_scale, inflation=True, pitch=None):
    """Outputs [B, H, D, N]: contiguous, or the [..., :N] views of rows of `pitch` elements whose
    padding holds PAD_BITS (run_gpu.rows keeps the whole padded buffers)."""
    B, N, H, D = g["q"].shape
    P = N if pitch is None else pitch
    rows = [torch.full((B, H, D, P), PAD_BITS, dtype=torch.int16, device=DEV).view(g["q"].dtype)
            for _ in range(3)]
    outs = [r[..., :N] for r in rows]
    run_gpu.rows = rows
    infl = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV) \
        if inflation else None
    qr.qkrope_cam_prep(g["q"], g["k"], g["v"], g["proj_q"], g["proj_kv"], g["rope_cos"],
                       g["rope_sin"], k_scale, q_out=outs[0], k_out=outs[1], v_out=outs[2],
                       inflation_sq=infl)
    return outs, infl


def check(name, outs, infl, ref):
    for o, r, n in zip(outs, ref[:3], ("q", "k", "v")):
        assert_cam_close(o, r, f"{name} {n}")
    if infl is not None:
        assert_inflation_close(infl, ref[3], f"{name} inflation_sq")


CASES = [
    # (B, N, H, D, act): what the case exercises
    (2, 200, 5, 64, "bf16"),    # 4 tiles with an 8-token tail, 16-byte stores, groups of 3 + 2
    (1, 130, 3, 128, "bf16"),   # N % 8 = 2: element stores; 1024-lane workgroups
    (2, 64, 4, 256, "bf16"),    # two chunks per lane, exactly one tile
    (1, 77, 2, 8, "bf16"),      # one lane per token
    (1, 1, 1, 16, "bf16"),      # a single token
    (3, 65, 7, 24, "bf16"),     # 3 chunks in 4-lane groups; a 1-token tail tile
    (1, 100, 6, 200, "bf16"),   # 25 chunks: two per lane, 13 of 16 lanes busy
    (2, 136, 4, 64, "f16"),     # binary16 activations and outputs
    (1, 96, 9, 32, "bf16"),     # 9 heads in 3 groups of 3
    (2, 18480 // 20, 20, 64, "bf16"),   # one frame of the SANA-WM grid, all 20 heads
]


@pytest.mark.parametrize("B,N,H,D,act", CASES)
def test_cam_matches_oracle(B, N, H, D, act):
    w = workload(B, N, H, D, act, seed=B * 1000 + N + H + D)
    print(f"\ncam parity {w.name}", flush=True)
    inp = wl.cam_inputs(w)
    outs, infl = run_gpu(gpu_inputs(inp), w.k_scale)
    torch.cuda.synchronize()
    ref = oracle.cam_prep(inp["q"], inp["k"], inp["v"], inp["proj_q"], inp["proj_kv"],
                          inp["rope_cos"], inp["rope_sin"], w.k_scale)
    check(w.name, outs, infl, ref)


# (tensor, b, n, h, d, 16-bit pattern) planted per activation format: NaNs of both signs (quiet,
# and the ones next to the infinities), -inf and -0 where ReLU applies
SPECIAL_SITES = {
    "bf16": [("q", 0, 5, 1, 3, 0xFFC0), ("q", 1, 70, 3, 40, 0x7FC0), ("q", 0, 135, 0, 63, 0xFF81),
             ("k", 0, 9, 2, 0, 0xFF81), ("k", 1, 64, 1, 17, 0x7F81), ("k", 1, 0, 3, 62, 0xFFC0),
             ("v", 0, 100, 0, 6, 0xFFC0), ("v", 1, 127, 2, 33, 0x7FC0),
             ("q", 0, 7, 0, 4, 0xFF80), ("k", 1, 8, 1, 9, 0xFF80), ("q", 0, 10, 0, 0, 0x8000)],
    "f16": [("q", 0, 5, 1, 3, 0xFE00), ("q", 1, 70, 3, 40, 0x7E00), ("q", 0, 135, 0, 63, 0xFC01),
            ("k", 0, 9, 2, 0, 0xFC01), ("k", 1, 64, 1, 17, 0x7C01), ("k", 1, 0, 3, 62, 0xFE00),
            ("v", 0, 100, 0, 6, 0xFE00), ("v", 1, 127, 2, 33, 0x7E00),
            ("q", 0, 7, 0, 4, 0xFC00), ("k", 1, 8, 1, 9, 0xFC00), ("q", 0, 10, 0, 0, 0x8000)],
}


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_cam_nan_and_special_inputs(act):
    """NaNs of either sign pass ReLU as the oracle's (PyTorch's) ReLU passes them: each makes
    the four output channels of its projection group NaN, and a NaN key head makes its
    inflation_sq NaN; -inf and -0 rectify to 0. NaN positions must be the oracle's exactly and
    every other value matches it to the usual tolerance."""
    w = workload(2, 136, 4, 64, act, seed=77)
    print(f"\ncam special values {w.name}", flush=True)
    inp = wl.cam_inputs(w)
    for name, b, n, h, d, bits in SPECIAL_SITES[act]:
        inp[name].view(torch.int16)[b, n, h, d] = bits - 65536 if bits >= 32768 else bits
    outs, infl = run_gpu(gpu_inputs(inp), w.k_scale)
    torch.cuda.synchronize()
    ref = oracle.cam_prep(inp["q"], inp["k"], inp["v"], inp["proj_q"], inp["proj_kv"],
                          inp["rope_cos"], inp["rope_sin"], w.k_scale)
    # three NaN groups of four channels in each tensor (Q's and K's -inf are rectified), and
    # three NaN keys
    assert [int(np.isnan(r).sum()) for r in ref] == [12, 12, 8, 3]
    for o, r, n in zip(list(outs) + [infl], ref, ("q", "k", "v", "inflation_sq")):
        g = to_f64(o).reshape(r.shape)
        assert np.array_equal(np.isnan(g), np.isnan(r)), f"{n}: NaN positions differ"
        keep_gpu = torch.where(torch.isnan(o), torch.zeros_like(o), o)
        keep_ref = np.where(np.isnan(r), 0.0, r)
        if n == "inflation_sq":
            assert_inflation_close(keep_gpu, keep_ref, f"{w.name} {n}")
        else:
            assert_cam_close(keep_gpu, keep_ref, f"{w.name} {n}")


def test_cam_hand_case_on_gpu():
    """The oracle's hand-worked single-head case, padded to head_dim 8 with a second group of
    four channels that the identity-like parts of the matrices leave alone."""
    x = torch.tensor([1.0, -2.0, 3.0, 4.0, 0.5, 0.25, -1.0, 2.0], dtype=torch.bfloat16)
    x = x.view(1, 1, 1, 8).to(DEV)
    pq = torch.tensor([[0, 1, 0, 0], [0, 0, 1, 0], [0, 0, 0, 1], [1, 0, 0, 0]],
                      dtype=torch.float32).view(1, 1, 4, 4).to(DEV)
    pkv = torch.diag(torch.tensor([2.0, 1.0, 1.0, 1.0])).view(1, 1, 4, 4).to(DEV)
    c = torch.tensor([[0.0, 1.0, 1.0, 1.0]], device=DEV)
    s = torch.tensor([[1.0, 0.0, 0.0, 0.0]], device=DEV)
    g = dict(q=x, k=x, v=x, proj_q=pq, proj_kv=pkv, rope_cos=c, rope_sin=s)
    outs, infl = run_gpu(g, 0.5)
    torch.cuda.synchronize()
    assert outs[0].float().cpu().view(8)[:4].tolist() == [-3.0, 0.0, 4.0, 1.0]
    assert outs[1].float().cpu().view(8)[:4].tolist() == [0.0, 1.0, 1.5, 2.0]
    assert outs[2].float().cpu().view(8)[:4].tolist() == [2.0, 2.0, 3.0, 4.0]
    # inflation over all 8 channels: second group of K: ReLU -> [0.5, 0.25, 0, 2] * 0.5,
    # diag(2,1,1,1) doubles its first channel
    a = 0.5 * np.array([1, 0, 3, 4, 0.5, 0.25, 0, 2.0])
    p = a * np.array([2, 1, 1, 1, 2, 1, 1, 1.0])
    assert infl.cpu().item() == pytest.approx((p @ p) / (a @ a), rel=2 ** -20)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("w", [wl.CAM_PREP_S18480, wl.CAM_PREP_S18432, wl.CAM_PREP_S18480_P18496],
                         ids=lambda w: w.name)
def test_cam_full_shape_every_token(w):
    """The SANA-WM shapes as bench.py runs them (2 x 18480 tokens, 20 heads of 64; 2 x 18432,
    whose output rows start on 128-byte lines; and 2 x 18480 into rows padded to 18496): every
    output of one launch against the oracle."""
    print(f"\ncam full shape {w.name}", flush=True)
    inp = wl.cam_inputs(w)
    g = gpu_inputs(inp)
    outs, infl = run_gpu(g, w.k_scale, pitch=w.out_pitch)
    torch.cuda.synchronize()
    ref = oracle.cam_prep(inp["q"], inp["k"], inp["v"], inp["proj_q"], inp["proj_kv"],
                          inp["rope_cos"], inp["rope_sin"], w.k_scale)
    check(w.name, outs, infl, ref)
    assert all(torch.isfinite(o.float()).all().item() for o in outs)
    assert torch.isfinite(infl).all().item()


@pytest.mark.parametrize("B,N,H,D,pitch,act", [
    (2, 200, 3, 64, 256, "bf16"),     # pitch a multiple of 64: rows on 128-byte lines
    (2, 200, 3, 64, 203, "bf16"),     # odd pitch: element stores
    (1, 130, 2, 128, 136, "bf16"),    # N % 8 != 0, pitch % 8 == 0: 16-byte stores on whole tiles
    (2, 150, 3, 64, 150, "bf16"),     # pitch == N: the contiguous layout
    (1, 100, 2, 256, 128, "bf16"),    # four chunks per lane: stores as each tensor is gathered
    (2, 136, 4, 64, 192, "f16"),      # binary16 activations and outputs
])
def test_cam_padded_output_rows(B, N, H, D, pitch, act):
    """Outputs with a row pitch above num_tokens: the same bits as contiguous outputs, the oracle's
    values, and the padding between N and the pitch untouched."""
    w = workload(B, N, H, D, act=act, seed=41)
    inp = wl.cam_inputs(w)
    g = gpu_inputs(inp)
    dense, infl = run_gpu(g, w.k_scale)
    padded, infl_p = run_gpu(g, w.k_scale, pitch=pitch)
    rows = run_gpu.rows
    torch.cuda.synchronize()
    for a, b in zip(dense, padded):
        assert torch.equal(a.view(torch.int16), b.contiguous().view(torch.int16))
    assert torch.equal(infl, infl_p)
    for r in rows:
        pad = r.view(torch.int16)[..., N:]
        assert bool((pad == PAD_BITS).all()), "padding written"
    ref = oracle.cam_prep(inp["q"], inp["k"], inp["v"], inp["proj_q"], inp["proj_kv"],
                          inp["rope_cos"], inp["rope_sin"], w.k_scale)
    check(w.name + f"_pitch{pitch}", [p.contiguous() for p in padded], infl_p, ref)


def test_cam_strided_rows_no_inflation_and_repeatability():
    """Padded token strides give the same bits as dense rows; inflation_sq=None changes no
    other output; two launches agree bit for bit."""
    w = workload(2, 150, 3, 64, seed=31)
    inp = gpu_inputs(wl.cam_inputs(w))
    dense, infl = run_gpu(inp, w.k_scale)
    B, N, H, D = inp["q"].shape
    padded = dict(inp)
    for name, extra in (("q", 8), ("k", 24), ("v", 64)):
        buf = torch.zeros((B, N, H * D + extra), dtype=inp[name].dtype, device=DEV)
        buf[:, :, :H * D] = inp[name].reshape(B, N, H * D)
        padded[name] = buf[:, :, :H * D].view(B, N, H, D)
    strided, _ = run_gpu(padded, w.k_scale, inflation=False)
    again, infl2 = run_gpu(inp, w.k_scale)
    torch.cuda.synchronize()
    for a, b, c in zip(dense, strided, again):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    assert torch.equal(infl, infl2)


@pytest.mark.parametrize("B,N,H", [(0, 10, 2), (2, 0, 2), (2, 10, 0)])
def test_cam_empty_is_noop(B, N, H):
    D = 64
    x = torch.zeros((B, N, H, D), dtype=torch.bfloat16, device=DEV)
    P = torch.zeros((B, N, 4, 4), dtype=torch.float32, device=DEV)
    t = torch.zeros((N, D // 2), dtype=torch.float32, device=DEV)
    outs = [torch.zeros((B, H, D, N), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    infl = torch.zeros((B, H, N), dtype=torch.float32, device=DEV)
    qr.qkrope_cam_prep(x, x, x, P, P, t, t, 1.0, q_out=outs[0], k_out=outs[1], v_out=outs[2],
                       inflation_sq=infl)
    torch.cuda.synchronize()


def test_cam_argument_errors():
    h = qr._handle_for(torch.device(DEV))
    L = qr.lib()
    B, N, H, D = 1, 16, 2, 64
    x = torch.zeros((B, N, H, D + 8), dtype=torch.bfloat16, device=DEV)
    P = torch.zeros((B, N, 4, 4), dtype=torch.float32, device=DEV)
    t = torch.zeros((N, 128), dtype=torch.float32, device=DEV)
    o = torch.zeros((3, B * H * (D + 8) * N + 64), dtype=torch.bfloat16, device=DEV)
    infl = torch.zeros(B * H * N, dtype=torch.float32, device=DEV)
    s = 0

    def call(D_, xs=None, q_out=None, act=qr.QKROPE_DTYPE_BF16, stride=H * (D + 8), pitch=N):
        xp = x.data_ptr() if xs is None else xs
        return L.qkrope_cam_prep(h, xp, x.data_ptr(), x.data_ptr(), act, P.data_ptr(),
                                 P.data_ptr(), t.data_ptr(), t.data_ptr(), 1.0, B, N, H, D_,
                                 stride, stride, stride,
                                 o[0].data_ptr() if q_out is None else q_out,
                                 o[1].data_ptr(), o[2].data_ptr(), pitch, infl.data_ptr(), s)

    assert call(64) == qr.QKROPE_OK
    assert call(6) == qr.QKROPE_ERR_INVALID            # not a multiple of 4
    assert call(12) == qr.QKROPE_ERR_UNSUPPORTED       # multiple of 4, not of 8
    assert call(264, stride=H * 264) == qr.QKROPE_ERR_UNSUPPORTED   # beyond 256
    assert call(64, act=qr.QKROPE_DTYPE_F32) == qr.QKROPE_ERR_INVALID
    assert call(64, xs=x.data_ptr() + 2) == qr.QKROPE_ERR_UNSUPPORTED   # misaligned q
    assert call(64, stride=H * 64 - 8) == qr.QKROPE_ERR_INVALID          # rows too short
    assert call(64, q_out=x.data_ptr()) == qr.QKROPE_ERR_INVALID         # output over q
    assert call(64, q_out=o[1].data_ptr() + 64) == qr.QKROPE_ERR_INVALID  # outputs overlap
    assert call(64, pitch=N - 1) == qr.QKROPE_ERR_INVALID                 # rows shorter than N
    assert call(64, pitch=1 << 31) == qr.QKROPE_ERR_UNSUPPORTED
    torch.cuda.synchronize()


def test_cam_graph_replay():
    """Captured in a HIP graph and replayed three times, with eager work between the replays;
    every replay matches the eager launch bit for bit."""
    w = workload(2, 192, 4, 64, seed=41)
    inp = gpu_inputs(wl.cam_inputs(w))
    eager, einfl = run_gpu(inp, w.k_scale)
    B, N, H, D = inp["q"].shape
    outs = [torch.empty_like(e) for e in eager]
    infl = torch.empty_like(einfl)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            qr.qkrope_cam_prep(inp["q"], inp["k"], inp["v"], inp["proj_q"], inp["proj_kv"],
                               inp["rope_cos"], inp["rope_sin"], w.k_scale, q_out=outs[0],
                               k_out=outs[1], v_out=outs[2], inflation_sq=infl)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        infl.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, outs):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep}"
        assert torch.equal(einfl, infl), f"replay {rep}"
