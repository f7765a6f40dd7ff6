"""Pins for the oracle's camera prologue (vLLM-Omni "vllm_omni.diffusion.models.sana_wm.ucpe"
page, cam_prep_func): ReLU, K scale, per-token 4x4 ray projection, interleaved RoPE from
separate (N, D/2) cos/sin tables, (B, H, D, N) outputs and inflation_sq (B, H, N).

The page names the steps and shapes but not how they compose; the oracle's header states the
readings taken. Each test checks the oracle against something other than its own loops: a
hand-worked case (tests/golden/hand_cases.json) built so that the other orders, a transposed
matrix or the opposite rotation sign give different numbers; the same composition written with
library primitives (a block-diagonal matrix from np.kron, RoPE as complex multiplication);
invariants (orthogonal P keeps norms, c*I inflates by c^2, K scale is linear); and the already
pinned table form, which P = I must reduce to.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def bf16_exact(x):
    b = oracle.bf16_encode(np.asarray(x, np.float64))
    assert np.array_equal(oracle.bf16_decode(b), np.asarray(x, np.float64))
    return b


def rand_bits(rng, shape, sigma=1.0):
    return oracle.bf16_encode(rng.standard_normal(shape) * sigma)


def decode(bits):
    return oracle.bf16_decode(bits)


def eye_proj(B, N):
    return np.broadcast_to(np.eye(4, dtype=np.float32), (B, N, 4, 4)).copy()


def zero_angle_tables(N, D):
    return np.ones((N, D // 2), np.float32), np.zeros((N, D // 2), np.float32)


def angle_tables(rng, N, D):
    theta = rng.uniform(-np.pi, np.pi, (N, D // 2))
    return np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)


def random_proj(rng, B, N, scale=0.5):
    return (np.eye(4) + scale * rng.standard_normal((B, N, 4, 4))).astype(np.float32)


def reference_by_primitives(x, P, cos, sin, relu, scale, grouped=False):
    """The stated composition written with library primitives, per (b, n, h): PyTorch's ReLU
    (the page presents cam_prep_func as the native equivalent of a PyTorch module), a
    block-diagonal kron(I, P) matmul (grouped: the [D/4, 4] groups times P^T, which keeps a NaN
    inside its group where the zeros of kron(I, P) would spread it), then RoPE as
    multiplication of complex pairs by cos + i sin. x: fp64 [B, N, H, D]. Returns fp64
    [B, H, D, N] and |p|^2 / |a|^2 [B, H, N] (1 where |a| = 0)."""
    B, N, H, D = x.shape
    a = scale * (torch.relu(torch.from_numpy(x)).numpy() if relu else x)
    out = np.empty((B, H, D, N))
    infl = np.empty((B, H, N))
    for b in range(B):
        for n in range(N):
            M = np.kron(np.eye(D // 4), P[b, n].astype(np.float64))
            rot = cos[n].astype(np.float64) + 1j * sin[n].astype(np.float64)
            for h in range(H):
                p = ((a[b, n, h].reshape(D // 4, 4) @ P[b, n].astype(np.float64).T).ravel()
                     if grouped else M @ a[b, n, h])
                z = (p[0::2] + 1j * p[1::2]) * rot
                out[b, h, 0::2, n] = z.real
                out[b, h, 1::2, n] = z.imag
                na = a[b, n, h] @ a[b, n, h]
                infl[b, h, n] = 1.0 if na == 0 else (p @ p) / na
    return out, infl


def test_cam_hand_case():
    g = GOLDEN["cam_prep_one_head"]
    x = bf16_exact(np.array(g["x"]).reshape(1, 1, 1, 4))
    pq = np.array(g["proj_q"], np.float32).reshape(1, 1, 4, 4)
    pkv = np.array(g["proj_kv"], np.float32).reshape(1, 1, 4, 4)
    c = np.array([g["cos"]], np.float32)
    s = np.array([g["sin"]], np.float32)
    qo, ko, vo, infl = oracle.cam_prep(x, x, x, pq, pkv, c, s, g["k_scale"])
    np.testing.assert_array_equal(qo.ravel(), g["q_out"])
    np.testing.assert_array_equal(ko.ravel(), g["k_out"])
    np.testing.assert_array_equal(vo.ravel(), g["v_out"])
    assert infl.ravel()[0] == pytest.approx(g["inflation_sq"], rel=1e-15)


def test_cam_identity_is_relu_scale_and_layout():
    """P = I and zero angles leave ReLU (Q), k_scale * ReLU (K) and V, moved to [B, H, D, N]."""
    rng = np.random.default_rng(11)
    B, N, H, D = 2, 5, 3, 8
    q, k, v = (rand_bits(rng, (B, N, H, D)) for _ in range(3))
    c, s = zero_angle_tables(N, D)
    qo, ko, vo, infl = oracle.cam_prep(q, k, v, eye_proj(B, N), eye_proj(B, N), c, s, 0.25)
    t = (0, 2, 3, 1)
    np.testing.assert_array_equal(qo, np.maximum(decode(q), 0).transpose(t))
    np.testing.assert_array_equal(ko, 0.25 * np.maximum(decode(k), 0).transpose(t))
    np.testing.assert_array_equal(vo, decode(v).transpose(t))
    np.testing.assert_allclose(infl, 1.0, rtol=1e-15)


def test_cam_matches_library_primitives():
    """Random per-token matrices and angles, two batches (tables are indexed by n only)."""
    rng = np.random.default_rng(12)
    B, N, H, D = 2, 7, 3, 16
    q, k, v = (rand_bits(rng, (B, N, H, D)) for _ in range(3))
    pq, pkv = random_proj(rng, B, N), random_proj(rng, B, N)
    c, s = angle_tables(rng, N, D)
    ks = 0.125 / np.sqrt(924.0)
    qo, ko, vo, infl = oracle.cam_prep(q, k, v, pq, pkv, c, s, ks)
    rq, _ = reference_by_primitives(decode(q), pq, c, s, True, 1.0)
    rk, rinfl = reference_by_primitives(decode(k), pkv, c, s, True, ks)
    rv, _ = reference_by_primitives(decode(v), pkv, c, s, False, 1.0)
    np.testing.assert_allclose(qo, rq, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ko, rk, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(vo, rv, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(infl, rinfl, rtol=1e-13)


def test_cam_orthogonal_projection_keeps_norms():
    """An orthogonal P and a rotation keep every head vector's norm: inflation 1, |y| = |a|."""
    rng = np.random.default_rng(13)
    B, N, H, D = 1, 6, 2, 12
    k = rand_bits(rng, (B, N, H, D))
    Q = np.stack([np.linalg.qr(rng.standard_normal((4, 4)))[0] for _ in range(N)])
    P = Q.astype(np.float32).reshape(B, N, 4, 4)
    theta = rng.uniform(-np.pi, np.pi, (N, D // 2))
    c, s = np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)
    _, ko, _, infl = oracle.cam_prep(k, k, k, eye_proj(B, N), P, c, s, 1.0)
    a = np.maximum(decode(k), 0)
    na = np.sqrt((a ** 2).sum(-1))                      # [B, N, H]
    ny = np.sqrt((ko ** 2).sum(2)).transpose(0, 2, 1)   # [B, N, H]
    # P is orthogonal only to float32 rounding, and so is cos^2 + sin^2 = 1
    np.testing.assert_allclose(ny, na, rtol=1e-6)
    np.testing.assert_allclose(infl, 1.0, rtol=1e-6)


def test_cam_scaled_identity_inflates_by_square():
    rng = np.random.default_rng(14)
    B, N, H, D = 1, 4, 2, 8
    k = rand_bits(rng, (B, N, H, D))
    P = (3.0 * eye_proj(B, N)).astype(np.float32)
    c, s = zero_angle_tables(N, D)
    _, ko, vo, infl = oracle.cam_prep(k, k, k, eye_proj(B, N), P, c, s, 0.5)
    np.testing.assert_allclose(infl, 9.0, rtol=1e-15)
    np.testing.assert_array_equal(ko, 1.5 * np.maximum(decode(k), 0).transpose(0, 2, 3, 1))
    np.testing.assert_array_equal(vo, 3.0 * decode(k).transpose(0, 2, 3, 1))


def test_cam_k_scale_is_linear_and_inflation_invariant():
    rng = np.random.default_rng(15)
    B, N, H, D = 1, 5, 2, 8
    q, k, v = (rand_bits(rng, (B, N, H, D)) for _ in range(3))
    pq, pkv = random_proj(rng, B, N), random_proj(rng, B, N)
    c, s = angle_tables(rng, N, D)
    _, k1, _, i1 = oracle.cam_prep(q, k, v, pq, pkv, c, s, 1.0)
    _, k2, _, i2 = oracle.cam_prep(q, k, v, pq, pkv, c, s, 0.375)
    np.testing.assert_allclose(k2, 0.375 * k1, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(i2, i1, rtol=1e-14)


def test_cam_all_negative_head():
    """ReLU of an all-negative head is zero: Q and K outputs vanish, inflation_sq reads 1."""
    B, N, H, D = 1, 1, 2, 4
    x = bf16_exact(np.array([-1.0, -2.0, -0.5, -4.0, 1.0, -2.0, 3.0, 0.5]).reshape(B, N, H, D))
    P = (2.0 * eye_proj(B, N)).astype(np.float32)
    c, s = zero_angle_tables(N, D)
    qo, ko, vo, infl = oracle.cam_prep(x, x, x, P, P, c, s, 1.0)
    assert np.all(qo[0, 0] == 0) and np.all(ko[0, 0] == 0)
    assert infl[0, 0, 0] == 1.0 and infl[0, 1, 0] == pytest.approx(4.0, rel=1e-15)
    np.testing.assert_array_equal(vo[0, 0, :, 0], 2.0 * decode(x)[0, 0, 0])


@pytest.mark.filterwarnings("ignore:invalid value encountered")
def test_cam_nan_propagates_like_library_relu():
    """A NaN of either sign, planted into q, k and v, passes through ReLU as PyTorch's does:
    the four channels of its projection group come out NaN (in every rotation pair of the
    group), inflation_sq of a key head holding one is NaN, and every other output equals the
    NaN-free run. The bf16 patterns include the NaNs next to the infinities (0x7F81, 0xFF81)
    and the quiet ones (0x7FC0, 0xFFC0)."""
    rng = np.random.default_rng(19)
    B, N, H, D = 2, 5, 3, 16
    q, k, v = (rand_bits(rng, (B, N, H, D)) for _ in range(3))
    pq, pkv = random_proj(rng, B, N), random_proj(rng, B, N)
    c, s = angle_tables(rng, N, D)
    ks = 0.125
    clean = oracle.cam_prep(q, k, v, pq, pkv, c, s, ks)
    plant = {  # tensor -> [(b, n, h, d, bits)]
        "q": [(0, 1, 0, 3, 0xFFC0), (1, 4, 2, 12, 0x7FC0), (1, 0, 1, 5, 0xFF81)],
        "k": [(0, 2, 1, 0, 0xFF81), (1, 3, 0, 9, 0x7F81), (0, 0, 2, 15, 0xFFC0)],
        "v": [(1, 1, 1, 6, 0xFFC0), (0, 4, 0, 1, 0x7FC0)],
    }
    x = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
    for name, sites in plant.items():
        for b, n, h, d, bits in sites:
            x[name][b, n, h, d] = bits
    qo, ko, vo, infl = oracle.cam_prep(x["q"], x["k"], x["v"], pq, pkv, c, s, ks)
    rq, _ = reference_by_primitives(decode(x["q"]), pq, c, s, True, 1.0, grouped=True)
    rk, rinfl = reference_by_primitives(decode(x["k"]), pkv, c, s, True, ks, grouped=True)
    rv, _ = reference_by_primitives(decode(x["v"]), pkv, c, s, False, 1.0, grouped=True)
    for got, ref, cl, name in ((qo, rq, clean[0], "q"), (ko, rk, clean[1], "k"),
                               (vo, rv, clean[2], "v")):
        want_nan = np.zeros(got.shape, bool)
        for b, n, h, d, _ in plant[name]:
            g = d // 4 * 4
            want_nan[b, h, g:g + 4, n] = True
        np.testing.assert_array_equal(np.isnan(got), want_nan, err_msg=name)
        np.testing.assert_array_equal(np.isnan(ref), want_nan, err_msg=name)
        np.testing.assert_allclose(got[~want_nan], ref[~want_nan], rtol=1e-13, atol=1e-14)
        np.testing.assert_array_equal(got[~want_nan], cl[~want_nan])
    want_nan = np.zeros(infl.shape, bool)
    for b, n, h, _, _ in plant["k"]:
        want_nan[b, h, n] = True
    np.testing.assert_array_equal(np.isnan(infl), want_nan)
    np.testing.assert_array_equal(np.isnan(rinfl), want_nan)
    np.testing.assert_array_equal(infl[~want_nan], clean[3][~want_nan])


def test_cam_relu_of_signed_zeros_and_infinities():
    """ReLU gives 0 for -0, +0, -inf and a negative subnormal and keeps a positive subnormal
    (P = I, zero angles: each value reaches the output unchanged). A +inf survives ReLU, and
    the projection then makes its whole group NaN (0 * inf in IEEE arithmetic), as the grouped
    library reference does."""
    B, N, H, D = 1, 1, 1, 12
    bits = np.array([0x8000, 0x0000, 0xFF80, 0xBF80, 0x3F80, 0x8001, 0x0001, 0x4000,
                     0x7F80, 0x3F80, 0xBF80, 0x0000], np.uint16).reshape(B, N, H, D)
    c, s = zero_angle_tables(N, D)
    P = eye_proj(B, N)
    qo, _, vo, _ = oracle.cam_prep(bits, bits, bits, P, P, c, s, 1.0)
    with np.errstate(invalid="ignore"):
        ref, _ = reference_by_primitives(decode(bits), P, c, s, True, 1.0, grouped=True)
    got = qo[0, 0, :, 0]
    np.testing.assert_array_equal(got[:8], [0, 0, 0, 0, 1.0, 0, decode(bits)[0, 0, 0, 6], 2.0])
    assert np.all(np.isnan(got[8:]))
    np.testing.assert_array_equal(got, ref[0, 0, :, 0])      # NaNs at the same places
    # V is not rectified: its -inf makes group 0 NaN, group 1 passes unchanged
    assert np.all(np.isnan(vo[0, 0, :4, 0]))
    np.testing.assert_array_equal(vo[0, 0, 4:8, 0], decode(bits)[0, 0, 0, 4:8])


def test_cam_identity_projection_equals_table_form():
    """With P = I and no negative inputs, the Q output is the table form's interleaved rotation
    with the same split tables and no norm (pinned in test_oracle_math.py)."""
    rng = np.random.default_rng(16)
    B, N, H, D = 1, 9, 3, 16
    q = oracle.bf16_encode(np.abs(rng.standard_normal((B, N, H, D))))
    c, s = angle_tables(rng, N, D)
    qo, _, _, _ = oracle.cam_prep(q, q, q, eye_proj(B, N), eye_proj(B, N), c, s, 1.0)
    tq, _ = oracle.run_table(q[0], q[0], None, None, c, 1e-6, interleaved=True,
                             norm_mode="none", sin_table=s)
    np.testing.assert_allclose(qo[0], tq.transpose(1, 2, 0), rtol=1e-15, atol=1e-300)


def test_cam_strided_rows_and_f16():
    rng = np.random.default_rng(17)
    B, N, H, D = 2, 3, 2, 8
    q, k, v = (rand_bits(rng, (B, N, H, D)) for _ in range(3))
    pq, pkv = random_proj(rng, B, N), random_proj(rng, B, N)
    c, s = angle_tables(rng, N, D)
    ref = oracle.cam_prep(q, k, v, pq, pkv, c, s, 0.5)
    pad = [np.zeros((B, N, H * D + 8), np.uint16) for _ in range(3)]
    for p_, x in zip(pad, (q, k, v)):
        p_[:, :, :H * D] = x.reshape(B, N, H * D)
    got = oracle.cam_prep(*pad, pq, pkv, c, s, 0.5, num_heads=H, head_dim=D)
    for a, b in zip(ref, got):
        np.testing.assert_array_equal(a, b)
    # binary16 activations holding the same values give the same result (these bf16 values of
    # magnitude < 8 are exact in binary16)
    h16 = [decode(x).astype(np.float16) for x in (q, k, v)]
    assert all(np.array_equal(h.astype(np.float64), decode(x)) for h, x in zip(h16, (q, k, v)))
    got16 = oracle.cam_prep(*h16, pq, pkv, c, s, 0.5)
    for a, b in zip(ref, got16):
        np.testing.assert_array_equal(a, b)


def test_cam_rejects_bad_shapes():
    rng = np.random.default_rng(18)
    B, N, H, D = 1, 2, 1, 6
    x = rand_bits(rng, (B, N, H, D))
    c, s = zero_angle_tables(N, D)
    with pytest.raises(ValueError):               # head_dim not a multiple of 4
        oracle.cam_prep(x, x, x, eye_proj(B, N), eye_proj(B, N), c, s, 1.0)
    x = rand_bits(rng, (B, N, H, 8))
    with pytest.raises(ValueError):               # tables of the wrong width
        oracle.cam_prep(x, x, x, eye_proj(B, N), eye_proj(B, N), c, s, 1.0)
    c8, s8 = zero_angle_tables(N, 8)
    with pytest.raises(ValueError):               # projections of the wrong shape
        oracle.cam_prep(x, x, x, eye_proj(B, N)[:, :, :3], eye_proj(B, N), c8, s8, 1.0)
