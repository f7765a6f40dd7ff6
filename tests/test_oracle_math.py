"""Pins for the oracle's arithmetic: RMSNorm, the two table pairings, 3D positions, YaRN.

Each test checks the oracle against something other than itself: a closed form, an invariant,
a special case that reduces to a textbook 1-D RoPE written with complex numbers, or a hand-worked
value (tests/golden/hand_cases.json). The tests are chosen so that a plausible slip in the oracle
(sum instead of mean, eps outside the root, a transposed pair, a wrong rotation sign, the wrong
position axis, a swapped YaRN blend) fails at least one of them.

Definitions followed:
  vLLM-Omni "vllm_omni.diffusion.layers.fused_qk_norm_rope" page, module contract;
  FlashInfer "flashinfer.norm.fused_qk_rmsnorm_rope" page, description and parameters.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def bf16_bits(x):
    """Exact bf16 bit patterns of values that are representable in bf16 (asserted)."""
    x = np.asarray(x, np.float64)
    b = oracle.bf16_encode(x)
    assert np.array_equal(oracle.bf16_decode(b), x), "test values must be bf16-exact"
    return b


def rand_bf16(rng, shape, sigma=1.0):
    return oracle.bf16_encode(rng.standard_normal(shape) * sigma)


def identity_table(T, R):
    return np.concatenate([np.ones((T, R // 2)), np.zeros((T, R // 2))], axis=1)


def angle_table(theta):
    """[T, R] fp64 table from angles [T, R/2] (the contract's [cos | sin] layout)."""
    return np.concatenate([np.cos(theta), np.sin(theta)], axis=1)


def ones_w(n):
    return bf16_bits(np.ones(n))


# --- RMSNorm -----------------------------------------------------------------------------------

def test_rmsnorm_hand_case():
    g = GOLDEN["rmsnorm_constant_row"]
    q = bf16_bits(np.array(g["x"]).reshape(1, 1, 4))
    qo, ko = oracle.run_table(q, q, ones_w(4), ones_w(4), identity_table(1, 4), g["eps"])
    np.testing.assert_allclose(qo.ravel(), g["expected"], rtol=1e-15)
    np.testing.assert_allclose(ko.ravel(), g["expected"], rtol=1e-15)


def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(1)
    q = rand_bf16(rng, (5, 3, 64))
    k2 = bf16_bits(oracle.bf16_decode(q) * 4.0)     # power-of-two scaling is exact in bf16
    tab = identity_table(5, 64)
    qo, ko = oracle.run_table(q, k2, ones_w(64), ones_w(64), tab, 0.0)
    # eps = 0, w = 1: each head has mean square exactly 1 (mean, not sum; square root taken)
    np.testing.assert_allclose((qo ** 2).mean(axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(qo, ko, rtol=1e-13)  # n(4x) = n(x)


def test_rmsnorm_eps_inside_root_and_weight_multiplies():
    d = float(oracle.bf16_decode(oracle.bf16_encode(np.array([1e-4])))[0])   # bf16 value near 1e-4
    q = bf16_bits(np.full((1, 1, 8), d))
    tab = identity_table(1, 8)
    qo, _ = oracle.run_table(q, q, ones_w(8), ones_w(8), tab, 1e-6)
    np.testing.assert_allclose(qo.ravel(), d / math.sqrt(d * d + 1e-6), rtol=1e-14)
    # weight 2 doubles the output, weight 0 zeroes it (w multiplies; it is not 1 + w)
    q2, k0 = oracle.run_table(q, q, bf16_bits(np.full(8, 2.0)), bf16_bits(np.zeros(8)), tab, 1e-6)
    np.testing.assert_allclose(q2, 2 * qo, rtol=1e-15)
    assert np.all(k0 == 0)
    # a zero row stays zero (no division by zero: eps is inside the root)
    z = bf16_bits(np.zeros((1, 1, 8)))
    zo, _ = oracle.run_table(z, z, ones_w(8), ones_w(8), tab, 1e-6)
    assert np.all(zo == 0)


def test_rmsnorm_constant_row_closed_form():
    for c in (0.5, -3.0, 1024.0):
        q = bf16_bits(np.full((1, 2, 16), c))
        qo, _ = oracle.run_table(q, q, ones_w(16), ones_w(16), identity_table(1, 16), 1e-6)
        np.testing.assert_allclose(qo, c / math.sqrt(c * c + 1e-6), rtol=1e-14)


def test_per_head_norm_is_per_head():
    rng = np.random.default_rng(2)
    q = oracle.bf16_decode(rand_bf16(rng, (2, 4, 32)))
    q_scaled = q.copy()
    q_scaled[:, 1] *= 8.0                             # scale one head only (exact)
    w = rand_bf16(rng, 32)
    tab = identity_table(2, 32)
    a, _ = oracle.run_table(bf16_bits(q), bf16_bits(q), w, w, tab, 0.0)
    b, _ = oracle.run_table(bf16_bits(q_scaled), bf16_bits(q), w, w, tab, 0.0)
    np.testing.assert_allclose(a, b, rtol=1e-13)     # every head, including the scaled one
    # the weight is indexed by d within the head: dividing it out leaves unit mean square heads
    unit = a / oracle.bf16_decode(w)
    np.testing.assert_allclose((unit ** 2).mean(axis=-1), 1.0, rtol=1e-13)


def test_across_heads_norm_relations():
    rng = np.random.default_rng(3)
    T, D = 3, 16
    one = rand_bf16(rng, (T, 1, D))
    w = rand_bf16(rng, D)
    tab = identity_table(T, D)
    # one head: across-heads == per-head
    a, _ = oracle.run_table(one, one, w, w, tab, 1e-6, norm_mode="per_head")
    b, _ = oracle.run_table(one, one, w, w, tab, 1e-6, norm_mode="across_heads")
    np.testing.assert_allclose(a, b, rtol=1e-14)
    # H identical heads: across-heads == per-head (weights tiled)
    rep = np.ascontiguousarray(np.repeat(one, 4, axis=1))
    c, _ = oracle.run_table(rep, rep, w, w, tab, 1e-6, norm_mode="per_head")
    d, _ = oracle.run_table(rep, rep, np.tile(w, 4), np.tile(w, 4), tab, 1e-6,
                            norm_mode="across_heads")
    np.testing.assert_allclose(c, d, rtol=1e-14)
    # across-heads: mean square over the whole row is 1 (eps 0, w 1), not per head
    x = rand_bf16(rng, (T, 3, D))
    e, _ = oracle.run_table(x, x, ones_w(3 * D), ones_w(3 * D), tab, 0.0, norm_mode="across_heads")
    np.testing.assert_allclose((e.reshape(T, -1) ** 2).mean(axis=1), 1.0, rtol=1e-13)
    assert not np.allclose((e ** 2).mean(axis=-1), 1.0)


# --- table-form rotation -----------------------------------------------------------------------

def test_position_zero_is_identity():
    rng = np.random.default_rng(4)
    q = rand_bf16(rng, (4, 2, 32))
    for inter in (False, True):
        qo, _ = oracle.run_table(q, q, None, None, identity_table(4, 32), 1e-6,
                                 interleaved=inter, norm_mode="none")
        np.testing.assert_array_equal(qo, oracle.bf16_decode(q))


def test_rotation_direction_quarter_turn():
    # theta = pi/2 turns (a, b) = (1, 0) into (0, 1): positive rotation, a' = a c - b s.
    tab = angle_table(np.full((1, 1), math.pi / 2))
    x = bf16_bits(np.array([1.0, 0.0]).reshape(1, 1, 2))
    qo, _ = oracle.run_table(x, x, None, None, tab, 0.0, interleaved=True, norm_mode="none")
    np.testing.assert_allclose(qo.ravel(), [0.0, 1.0], atol=1e-15)


def test_rope_hand_case_both_pairings():
    g = GOLDEN["rope_position_one"]
    x = bf16_bits(np.array(g["x"]).reshape(1, 1, 4))
    tab = angle_table(np.array([g["theta"]]))
    a, _ = oracle.run_table(x, x, None, None, tab, 0.0, interleaved=True, norm_mode="none")
    b, _ = oracle.run_table(x, x, None, None, tab, 0.0, interleaved=False, norm_mode="none")
    np.testing.assert_allclose(a.ravel(), g["interleaved"], rtol=1e-15, atol=1e-17)
    np.testing.assert_allclose(b.ravel(), g["half_split"], rtol=1e-15, atol=1e-17)


def test_pair_norm_preserved_and_partial_rotary():
    rng = np.random.default_rng(5)
    T, H, D, R = 6, 3, 32, 20
    q = rand_bf16(rng, (T, H, D))
    tab = angle_table(rng.uniform(-40, 40, (T, R // 2)))
    x = oracle.bf16_decode(q)
    for inter in (False, True):
        qo, _ = oracle.run_table(q, q, None, None, tab, 0.0, rotary_dim=R, interleaved=inter,
                                 norm_mode="none")
        if inter:
            a, b = np.arange(0, R, 2), np.arange(1, R, 2)
        else:
            a, b = np.arange(R // 2), np.arange(R // 2) + R // 2
        np.testing.assert_allclose(qo[..., a] ** 2 + qo[..., b] ** 2,
                                   x[..., a] ** 2 + x[..., b] ** 2, rtol=1e-12)
        np.testing.assert_array_equal(qo[..., R:], x[..., R:])   # beyond rotary_dim: untouched


def test_rotations_compose():
    rng = np.random.default_rng(6)
    T, D = 4, 16
    q = rand_bf16(rng, (T, 2, D))
    t1, t2 = rng.uniform(-3, 3, (T, D // 2)), rng.uniform(-3, 3, (T, D // 2))
    for inter in (False, True):
        once, _ = oracle.run_table(q, q, None, None, angle_table(t1 + t2), 0.0,
                                   interleaved=inter, norm_mode="none")
        half, _ = oracle.run_table(q, q, None, None, angle_table(t1), 0.0,
                                   interleaved=inter, norm_mode="none")
        # second step on fp64 values: rotate `half` by t2 with the complex form
        z = to_complex(half, inter)
        z2 = z * np.exp(1j * t2)[:, None, :]
        np.testing.assert_allclose(from_complex(z2, inter, D), once, atol=1e-12)


def test_halfsplit_is_permuted_interleaved():
    rng = np.random.default_rng(7)
    T, H, D = 5, 2, 24
    q = rand_bf16(rng, (T, H, D))
    w = rand_bf16(rng, D)
    tab = angle_table(rng.uniform(-10, 10, (T, D // 2)))
    perm = np.empty(D, int)                          # P(x)[2i] = x[i], P(x)[2i+1] = x[i + D/2]
    perm[0::2] = np.arange(D // 2)
    perm[1::2] = np.arange(D // 2) + D // 2
    qp = np.ascontiguousarray(q[..., perm])
    hs, _ = oracle.run_table(q, q, w, w, tab, 1e-6, interleaved=False)
    il, _ = oracle.run_table(qp, qp, np.ascontiguousarray(w[perm]), np.ascontiguousarray(w[perm]),
                             tab, 1e-6, interleaved=True)
    inv = np.argsort(perm)
    np.testing.assert_allclose(il[..., inv], hs, rtol=1e-14, atol=1e-15)


# --- an independent brute force with complex numbers -------------------------------------------

def to_complex(x, interleaved, R=None):
    R = x.shape[-1] if R is None else R
    if interleaved:
        return x[..., 0:R:2] + 1j * x[..., 1:R:2]
    return x[..., : R // 2] + 1j * x[..., R // 2: R]


def from_complex(z, interleaved, D):
    out = np.empty(z.shape[:-1] + (D,))
    R = 2 * z.shape[-1]
    if interleaved:
        out[..., 0:R:2], out[..., 1:R:2] = z.real, z.imag
    else:
        out[..., : R // 2], out[..., R // 2: R] = z.real, z.imag
    return out


def brute_table(x, w, theta, eps, R, interleaved, norm_mode):
    """Textbook RMSNorm then z * exp(i theta) per pair; pure numpy, independent of oracle.c."""
    T, H, D = x.shape
    if norm_mode == "per_head":
        n = x / np.sqrt((x ** 2).mean(axis=-1, keepdims=True) + eps) * w
    elif norm_mode == "across_heads":
        ms = (x.reshape(T, -1) ** 2).mean(axis=1)[:, None, None]
        n = x / np.sqrt(ms + eps) * w.reshape(H, D)
    else:
        n = x.copy()
    z = to_complex(n, interleaved, R) * np.exp(1j * theta)[:, None, :]
    out = n.copy()
    out[..., :R] = from_complex(z, interleaved, R)
    return out


@pytest.mark.parametrize("D,R,inter,mode", [(8, 8, True, "per_head"), (8, 8, False, "per_head"),
                                            (12, 6, True, "across_heads"),
                                            (16, 8, False, "none"), (6, 4, True, "per_head")])
def test_table_form_matches_brute_force(D, R, inter, mode):
    rng = np.random.default_rng(D * 100 + R)
    T, Hq, Hk = 4, 3, 2
    q, k = rand_bf16(rng, (T, Hq, D)), rand_bf16(rng, (T, Hk, D))
    wl = D if mode != "across_heads" else None
    wq = rand_bf16(rng, wl or Hq * D)
    wk = rand_bf16(rng, wl or Hk * D)
    theta = rng.uniform(-50, 50, (T, R // 2))
    qo, ko = oracle.run_table(q, k, wq, wk, angle_table(theta), 1e-5, rotary_dim=R,
                              interleaved=inter, norm_mode=mode)
    dq = oracle.bf16_decode
    np.testing.assert_allclose(qo, brute_table(dq(q), dq(wq), theta, 1e-5, R, inter, mode),
                               rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ko, brute_table(dq(k), dq(wk), theta, 1e-5, R, inter, mode),
                               rtol=1e-12, atol=1e-13)


def rand_f16(rng, shape, sigma=1.0):
    return (rng.standard_normal(shape) * sigma).astype(np.float16)


@pytest.mark.parametrize("D,R,inter,mode,tdt", [(8, 8, True, "per_head", np.float16),
                                                (16, 16, False, "per_head", np.float32),
                                                (12, 6, True, "across_heads", np.float32),
                                                (16, 8, False, "none", np.float16)])
def test_table_form_float16_matches_brute_force(D, R, inter, mode, tdt):
    # float16 activations and weights ("the activation dtype"); the table in float16 or float32
    rng = np.random.default_rng(D * 10 + R + 7)
    T, Hq, Hk = 4, 3, 2
    q, k = rand_f16(rng, (T, Hq, D)), rand_f16(rng, (T, Hk, D))
    wl = D if mode != "across_heads" else None
    wq, wk = (1 + 0.1 * rand_f16(rng, wl or Hq * D)).astype(np.float16), \
        (1 + 0.1 * rand_f16(rng, wl or Hk * D)).astype(np.float16)
    theta = rng.uniform(-50, 50, (T, R // 2))
    tab = angle_table(theta).astype(tdt)
    qo, ko = oracle.run_table(q, k, wq, wk, tab, 1e-5, rotary_dim=R, interleaved=inter,
                              norm_mode=mode)
    # the rounded table entries are not an exact unit phasor: multiply by c + i s as stored
    c, s = tab[:, : R // 2].astype(np.float64), tab[:, R // 2:].astype(np.float64)
    f = lambda a: a.astype(np.float64)
    for x, w, out in ((q, wq, qo), (k, wk, ko)):
        ref = brute_table(f(x), f(w), np.zeros((T, R // 2)), 1e-5, R, inter, mode)  # norm only
        z = to_complex(ref, inter, R) * (c + 1j * s)[:, None, :]
        ref[..., :R] = from_complex(z, inter, R)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_split_cos_sin_tables_match_brute_force():
    # separate [T, R/2] cosine and sine tables with their own (padded) token strides
    rng = np.random.default_rng(23)
    T, H, D, R = 5, 2, 16, 12
    q, k = rand_bf16(rng, (T, H, D)), rand_bf16(rng, (T, H, D))
    wq, wk = rand_bf16(rng, D), rand_bf16(rng, D)
    theta = rng.uniform(-9, 9, (T, R // 2))
    cos_t = np.zeros((T, R // 2 + 3))
    sin_t = np.zeros((T, R // 2 + 5))
    cos_t[:, : R // 2], sin_t[:, : R // 2] = np.cos(theta), np.sin(theta)
    cos_t[:, R // 2:], sin_t[:, R // 2:] = 7.0, -7.0       # padding the oracle must not read
    dq = oracle.bf16_decode
    for inter in (True, False):
        qo, ko = oracle.run_table(q, k, wq, wk, cos_t, 1e-6, rotary_dim=R, interleaved=inter,
                                  sin_table=sin_t)
        np.testing.assert_allclose(qo, brute_table(dq(q), dq(wq), theta, 1e-6, R, inter,
                                                   "per_head"), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ko, brute_table(dq(k), dq(wk), theta, 1e-6, R, inter,
                                                   "per_head"), rtol=1e-12, atol=1e-13)


# --- 3D form -----------------------------------------------------------------------------------

def rope1d_freqs(C, base):
    """Textbook 1-D RoPE frequencies base^(-(0, 2, 4, ...)/C)."""
    return base ** (-np.arange(0, C, 2, dtype=np.float64) / C)


def grid_order(ppf, pph, ppw):
    """(f, h, w) of every sequence index, enumerated frame-major (width fastest)."""
    return np.array(list(itertools.product(range(ppf), range(pph), range(ppw))))


def run3d(qkv, wq, wk, **kw):
    return oracle.run_3d(qkv, wq, wk, **kw)


@pytest.mark.parametrize("axis", [0, 1, 2])
@pytest.mark.parametrize("inter", [True, False])
def test_3d_single_axis_is_1d_rope_of_that_axis(axis, inter):
    ppf, pph, ppw, D, H = 3, 4, 5, 8, 2
    C = [0, 0, 0]
    C[axis] = D
    rng = np.random.default_rng(10 + axis)
    S = ppf * pph * ppw
    qkv = rand_bf16(rng, (S, 3 * H * D))
    q, k, v = run3d(qkv, None, None, ppf=ppf, pph=pph, ppw=ppw, num_frame_channels=C[0],
                    num_height_channels=C[1], num_width_channels=C[2], num_heads_q=H,
                    num_heads_k=H, num_heads_v=H, head_dim=D, base=10000.0,
                    interleave=inter, is_qk_norm=False)
    pos = grid_order(ppf, pph, ppw)[:, axis]
    theta = pos[:, None] * rope1d_freqs(D, 10000.0)[None, :]
    x = oracle.bf16_decode(qkv).reshape(S, 3, H, D)
    ref = from_complex(to_complex(x[:, 0], inter) * np.exp(1j * theta)[:, None, :], inter, D)
    np.testing.assert_allclose(q, ref, atol=1e-13)
    np.testing.assert_array_equal(v, x[:, 2])


def test_3d_equals_table_form_with_matching_table():
    ppf, pph, ppw = 2, 3, 4
    Cf, Ch, Cw, D, H = 4, 6, 6, 16, 3
    rng = np.random.default_rng(12)
    B, S = 2, ppf * pph * ppw
    qkv = rand_bf16(rng, (B * S, 3 * H * D))
    wq, wk = rand_bf16(rng, H * D), rand_bf16(rng, H * D)
    # matching table, built here from the textbook per-axis frequencies (concatenated)
    freqs = np.concatenate([rope1d_freqs(c, 10000.0) for c in (Cf, Ch, Cw)])
    axis_of = np.repeat([0, 1, 2], [Cf // 2, Ch // 2, Cw // 2])
    pos = np.tile(grid_order(ppf, pph, ppw), (B, 1))
    theta = pos[:, axis_of] * freqs[None, :]
    tab = angle_table(theta)
    x = oracle.bf16_decode(qkv).reshape(B * S, 3, H, D)
    for inter in (True, False):
        q, k, v = run3d(qkv, wq, wk, ppf=ppf, pph=pph, ppw=ppw, num_frame_channels=Cf,
                        num_height_channels=Ch, num_width_channels=Cw, num_heads_q=H,
                        num_heads_k=H, num_heads_v=H, head_dim=D, eps=1e-6, interleave=inter)
        qb = oracle.bf16_encode(x[:, 0])
        kb = oracle.bf16_encode(x[:, 1])
        tq, tk = oracle.run_table(qb, kb, wq, wk, tab, 1e-6, interleaved=inter,
                                  norm_mode="across_heads")
        np.testing.assert_allclose(q, tq, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(k, tk, rtol=1e-12, atol=1e-13)
        np.testing.assert_array_equal(v, x[:, 2])


def test_3d_batch_repeats_positions_and_token_offset_slices():
    ppf, pph, ppw, D, H = 2, 2, 3, 8, 1
    rng = np.random.default_rng(13)
    S = ppf * pph * ppw
    one = rand_bf16(rng, (S, 3 * H * D))
    two = np.ascontiguousarray(np.concatenate([one, one]))
    kw = dict(ppf=ppf, pph=pph, ppw=ppw, num_frame_channels=2, num_height_channels=2,
              num_width_channels=4, num_heads_q=H, num_heads_k=H, num_heads_v=H, head_dim=D)
    wq = rand_bf16(rng, H * D)
    q1, _, _ = run3d(one, wq, wq, **kw)
    q2, _, _ = run3d(two, wq, wq, **kw)
    np.testing.assert_array_equal(q2[:S], q1)
    np.testing.assert_array_equal(q2[S:], q1)          # token t and t + S share a position
    qs, _, _ = run3d(np.ascontiguousarray(two[S + 5:S + 9]), wq, wq, token_offset=S + 5, **kw)
    np.testing.assert_array_equal(qs, q2[S + 5:S + 9])


def test_3d_no_norm_flag_and_attention_factor():
    ppf, pph, ppw, D, H = 1, 2, 8, 16, 2
    rng = np.random.default_rng(14)
    S = ppf * pph * ppw
    qkv = rand_bf16(rng, (S, 3 * H * D))
    kw = dict(ppf=ppf, pph=pph, ppw=ppw, num_frame_channels=4, num_height_channels=4,
              num_width_channels=8, num_heads_q=H, num_heads_k=H, num_heads_v=H, head_dim=D)
    x = oracle.bf16_decode(qkv).reshape(S, 3, H, D)
    af = 1.0 + 0.1 * math.log(4.0)
    for inter in (True, False):
        q, k, _ = run3d(qkv, None, None, is_qk_norm=False, factor=4.0, low=1.0, high=3.0,
                        attention_factor=af, interleave=inter, **kw)
        za, zx = to_complex(q, inter), to_complex(x[:, 0], inter)
        np.testing.assert_allclose(np.abs(za), af * np.abs(zx), rtol=1e-13)
    # is_qk_norm=False ignores weights; position 0 then returns the input exactly
    q0, _, _ = run3d(np.ascontiguousarray(qkv[:1]), None, None, is_qk_norm=False, **kw)
    np.testing.assert_array_equal(q0[0], x[0, 0])


def yarn_probe(C_axis, j, pos_axis, factor, low, high, af, base=10000.0):
    """Angle and magnitude the oracle applies to pair j of a one-axis 3D problem at a position."""
    D = C_axis
    C = [0, 0, 0]
    C[pos_axis] = D
    grid = [1, 1, 1]
    grid[pos_axis] = 3
    S = 3
    x = np.zeros((S, 3 * D))
    x[:, 2 * j] = 1.0                                 # interleaved pair j = (2j, 2j+1) = (1, 0)
    qkv = bf16_bits(x)
    q, _, _ = run3d(qkv, None, None, ppf=grid[0], pph=grid[1], ppw=grid[2],
                    num_frame_channels=C[0], num_height_channels=C[1], num_width_channels=C[2],
                    num_heads_q=1, num_heads_k=1, num_heads_v=1, head_dim=D, base=base,
                    factor=factor, low=low, high=high, attention_factor=af, is_qk_norm=False)
    a, b = q[1, 0, 2 * j], q[1, 0, 2 * j + 1]         # sequence index 1 = position 1 on that axis
    return math.atan2(b, a), math.hypot(a, b)


def test_yarn_hand_values():
    g = GOLDEN["yarn_blend"]
    for case in g["cases"]:
        for axis in (0, 2):
            ang, mag = yarn_probe(case["C"], case["j"], axis, g["factor"], g["low"], g["high"], 1.25)
            assert ang == pytest.approx(case["omega_prime"], rel=1e-12)
            assert mag == pytest.approx(1.25, rel=1e-14)
    assert g["cases"][1]["omega_prime"] == pytest.approx(0.1975 / 31, rel=1e-15)


def test_yarn_special_cases():
    C = 16
    for j in range(C // 2):
        plain = rope1d_freqs(C, 10000.0)[j]
        # factor 1: plain RoPE
        assert yarn_probe(C, j, 1, 1.0, 0.0, 0.0, 1.0)[0] == pytest.approx(plain, rel=1e-13)
        # ramp 1 everywhere (low=-2, high=-1): frequencies divided by the factor, which is
        # plain RoPE at position p / factor (linear position interpolation)
        assert yarn_probe(C, j, 1, 4.0, -2.0, -1.0, 1.0)[0] == pytest.approx(plain / 4, rel=1e-13)
        # ramp 0 everywhere (low beyond the last pair): plain RoPE
        assert yarn_probe(C, j, 1, 4.0, C, C + 1.0, 1.0)[0] == pytest.approx(plain, rel=1e-13)


def test_3d_rejects_contract_violations():
    qkv = np.zeros((4, 3 * 8), np.uint16)
    kw = dict(ppf=1, pph=2, ppw=2, num_heads_q=1, num_heads_k=1, num_heads_v=1, head_dim=8)
    with pytest.raises(ValueError):                   # channels do not sum to head_dim
        run3d(qkv, None, None, num_frame_channels=2, num_height_channels=2,
              num_width_channels=2, is_qk_norm=False, **kw)
    with pytest.raises(ValueError):                   # odd channel count
        run3d(qkv, None, None, num_frame_channels=3, num_height_channels=3,
              num_width_channels=2, is_qk_norm=False, **kw)
    with pytest.raises(ValueError):                   # attention factor without YaRN
        run3d(qkv, None, None, num_frame_channels=2, num_height_channels=2,
              num_width_channels=4, is_qk_norm=False, attention_factor=2.0, **kw)


# --- per-token sums of squares (first phase of a head-sharded across-heads norm) --------------

def test_sumsq_closed_form_and_head_split_additivity():
    Hq, Hk, Hv, D, T = 4, 2, 3, 8, 6
    row = (Hq + Hk + Hv) * D
    const = np.tile(bf16_bits(np.r_[np.full(Hq * D, 0.5), np.full(Hk * D, -3.0),
                                    np.full(Hv * D, 100.0)]), (T, 1))
    s = oracle.sumsq_3d(const, num_heads_q=Hq, num_heads_k=Hk, num_heads_v=Hv, head_dim=D)
    np.testing.assert_array_equal(s, np.tile([Hq * D * 0.25, Hk * D * 9.0], (T, 1)))
    # shards holding 1 + 3 Q heads and 1 + 1 K heads: their sums add up to the whole row's
    rng = np.random.default_rng(29)
    x = rand_bf16(rng, (T, row)).reshape(T, Hq + Hk + Hv, D)
    full = oracle.sumsq_3d(x.reshape(T, row), num_heads_q=Hq, num_heads_k=Hk, num_heads_v=Hv,
                           head_dim=D)
    parts = []
    for qh, kh in (((0,), (4,)), ((1, 2, 3), (5,))):
        sx = np.ascontiguousarray(np.concatenate([x[:, list(qh)], x[:, list(kh)]], axis=1))
        parts.append(oracle.sumsq_3d(sx.reshape(T, -1), num_heads_q=len(qh),
                                     num_heads_k=len(kh), num_heads_v=0, head_dim=D))
    np.testing.assert_allclose(parts[0] + parts[1], full, rtol=1e-14)


def test_sumsq_is_what_the_across_heads_norm_averages():
    # one grid position (ppf = pph = ppw = 1): no rotation, unit weights, so the 3D form's Q
    # output is x / sqrt(sumsq / (Hq*D) + eps)
    Hq, Hk, Hv, D, T, eps = 3, 2, 1, 8, 5, 1e-3
    rng = np.random.default_rng(31)
    qkv = rand_bf16(rng, (T, (Hq + Hk + Hv) * D))
    ones_q, ones_k = bf16_bits(np.ones(Hq * D)), bf16_bits(np.ones(Hk * D))
    q, k, _ = oracle.run_3d(qkv, ones_q, ones_k, ppf=1, pph=1, ppw=1, num_frame_channels=D,
                            num_height_channels=0, num_width_channels=0, num_heads_q=Hq,
                            num_heads_k=Hk, num_heads_v=Hv, head_dim=D, eps=eps)
    s = oracle.sumsq_3d(qkv, num_heads_q=Hq, num_heads_k=Hk, num_heads_v=Hv, head_dim=D)
    x = oracle.bf16_decode(qkv)
    np.testing.assert_allclose(q.reshape(T, -1) * np.sqrt(s[:, :1] / (Hq * D) + eps),
                               x[:, : Hq * D], rtol=1e-13)
    np.testing.assert_allclose(k.reshape(T, -1) * np.sqrt(s[:, 1:] / (Hk * D) + eps),
                               x[:, Hq * D:(Hq + Hk) * D], rtol=1e-13)
