"""Seeded random sweep of the camera prologue (qkrope_cam_prep) on the GPU against the fp64 oracle.

Each case draws batch, token count (multiples of 8 or not, below and above one 64-token tile),
heads (groups of two and a lone last head), head_dim (any multiple of 8 up to 256: one or two
chunks per lane, lane groups that a head's chunks do not fill), bf16 or binary16, padded token
strides, general 4x4 matrices (not only rigid transforms), random angles and k_scale, and
inflation_sq present or not; every output element is compared at the criteria in parity.py.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from parity import assert_cam_close, assert_inflation_close

pytestmark = pytest.mark.gpu

qr = pytest.importorskip("qk_rmsnorm_rope_amd")
from qk_rmsnorm_rope_amd import workloads as wl  # noqa: E402

DEV = "cuda"
# QKROPE_SWEEP_CASES runs that many cases instead (same draws, more indices)
NCASES = int(os.environ.get("QKROPE_SWEEP_CASES", "200"))


def draw(i):
    rng = np.random.default_rng(7000 + i)
    B = int(rng.integers(1, 4))
    N = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 300)),
                        8 * int(rng.integers(1, 40))]))
    H = int(rng.integers(1, 8))
    D = 8 * int(rng.integers(1, 33))
    act = "f16" if rng.random() < 0.3 else "bf16"
    pads = [8 * int(rng.integers(0, 4)) for _ in range(3)]
    with_infl = bool(rng.random() < 0.8)
    k_scale = float(rng.choice([1.0, 0.125, float(rng.uniform(0.001, 2.0))]))
    sigma = float(rng.choice([1.0, 2.5]))
    return dict(B=B, N=N, H=H, D=D, act=act, pads=pads, with_infl=with_infl, k_scale=k_scale,
                sigma=sigma, seed=7100 + 10 * i)


def inputs(c):
    B, N, H, D = c["B"], c["N"], c["H"], c["D"]
    n = B * N * H * D
    xs = [wl.bf16_normal(c["seed"] + r, n, c["sigma"], c["act"]).view(B, N, H, D) for r in range(3)]
    rng = np.random.default_rng(c["seed"] + 5)
    P = [torch.from_numpy((np.eye(4) + 0.5 * rng.standard_normal((B, N, 4, 4))).astype(np.float32))
         for _ in range(2)]
    theta = rng.uniform(-np.pi, np.pi, (N, D // 2))
    cos = torch.from_numpy(np.cos(theta).astype(np.float32))
    sin = torch.from_numpy(np.sin(theta).astype(np.float32))
    return xs, P, cos, sin


def padded(x, pad):
    B, N, H, D = x.shape
    buf = torch.zeros((B, N, H * D + pad), dtype=x.dtype, device=DEV)
    buf[:, :, :H * D] = x.reshape(B, N, H * D).to(DEV)
    return buf[:, :, :H * D].view(B, N, H, D)


@pytest.mark.parametrize("i", range(NCASES))
def test_random_cam(i):
    c = draw(i)
    print(f"\ncam sweep case {i}: {c}", flush=True)
    xs, P, cos, sin = inputs(c)
    B, N, H, D = c["B"], c["N"], c["H"], c["D"]
    g = [padded(x, p) for x, p in zip(xs, c["pads"])]
    outs = [torch.full((B, H, D, N), float("nan"), dtype=xs[0].dtype, device=DEV) for _ in range(3)]
    infl = torch.full((B, H, N), float("nan"), device=DEV) if c["with_infl"] else None
    qr.qkrope_cam_prep(g[0], g[1], g[2], P[0].to(DEV), P[1].to(DEV), cos.to(DEV), sin.to(DEV),
                       c["k_scale"], q_out=outs[0], k_out=outs[1], v_out=outs[2],
                       inflation_sq=infl)
    torch.cuda.synchronize()
    ref = oracle.cam_prep(xs[0], xs[1], xs[2], P[0], P[1], cos, sin, c["k_scale"])
    for o, r, n in zip(outs, ref[:3], ("q", "k", "v")):
        assert_cam_close(o, r, f"case {i} {n}")
    if infl is not None:
        assert_inflation_close(infl, ref[3], f"case {i} inflation_sq")
