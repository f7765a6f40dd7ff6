"""Pins for the oracle's number formats (bf16 RNE encoder, OCP E4M3 encoder/decoder).

The FlashInfer fused_qk_rmsnorm_rope page (parameters output_fp8 / output_quant_scale /
v_quant_scale) asks for FP8 E4M3 outputs; the format itself is fixed by the OCP 8-bit floating
point specification (E4M3: bias 7, largest finite 448, no infinities, S.1111.111 = NaN). bf16 is
the top half of IEEE-754 binary32. These tests pin the oracle's encoders to those definitions and
to torch's own casts, independently of the oracle's arithmetic.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def test_e4m3_all_finite_codes_round_trip():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254                      # only 0x7F and 0xFF are NaN
    assert set(codes[~finite].tolist()) == {0x7F, 0xFF}
    back = oracle.e4m3_encode(vals[finite])
    np.testing.assert_array_equal(back, codes[finite])


def test_e4m3_format_constants():
    dec = oracle.e4m3_decode
    assert dec(np.uint8(0x7E)) == 448.0             # largest finite: 1.75 * 2^8
    assert dec(np.uint8(0x08)) == 2.0 ** -6         # smallest normal
    assert dec(np.uint8(0x01)) == 2.0 ** -9         # smallest subnormal
    assert dec(np.uint8(0x38)) == 1.0               # exponent field 7 = bias
    assert dec(np.uint8(0xB8)) == -1.0
    # the decoded finite codes are strictly increasing in sign-magnitude order
    pos = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    # ulp is 0.125 on [1, 2)
    assert dec(np.uint8(0x39)) - dec(np.uint8(0x38)) == 0.125


def test_e4m3_rounding_ties_to_even_and_saturation():
    enc = lambda x: int(oracle.e4m3_encode(np.array([x]))[0])
    assert enc(1.0625) == 0x38                      # midway 1 / 1.125 -> even mantissa (1.0)
    assert enc(1.1875) == 0x3A                      # midway 1.125 / 1.25 -> 1.25 (even)
    assert enc(1.0625 + 1e-9) == 0x39               # just above the tie rounds up
    assert enc(2.0 ** -10) == 0x00                  # half the smallest subnormal: tie to 0
    assert enc(3 * 2.0 ** -10) == 0x02              # 1.5 quanta -> 2 (even)
    assert enc(464.0) == 0x7E                       # above 448 saturates
    assert enc(1e9) == 0x7E and enc(-1e9) == 0xFE
    assert enc(math.inf) == 0x7E
    assert enc(-0.0) == 0x80 and enc(0.0) == 0x00
    assert enc(math.nan) == 0x7F


def test_e4m3_scale_multiplies():
    x = np.array([1.0, -3.0, 100.0])
    np.testing.assert_array_equal(oracle.e4m3_encode(x, 0.5), oracle.e4m3_encode(x * 0.5))
    assert oracle.e4m3_encode(np.array([2.0]), 0.5)[0] == 0x38   # 2 * 0.5 = 1


def test_e4m3_matches_torch_cast_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (0.01, 1.0, 30.0, 150.0)])
    x = x[np.abs(x) <= 448.0].astype(np.float32)
    # include every midpoint between neighbouring finite codes (exactly representable in fp32)
    pos = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids]).astype(np.float32)
    ours = oracle.e4m3_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(50000).astype(np.float32) * s
                        for s in (1e-40, 1e-5, 1.0, 1e30)])
    u = np.arange(0x3F800000, 0x3F800000 + (1 << 17), 7, dtype=np.uint64).astype(np.uint32)
    ties = u.view(np.float32)                       # includes exact bf16 midpoints (low half 0x8000)
    edge = np.array([3.3895314e38, 3.4e38, -3.4028235e38, 1e-45, -0.0, 0.0], np.float32)
    x = np.concatenate([x, ties, edge]).astype(np.float32)
    ours = oracle.bf16_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_rounds_from_fp64_directly():
    # 1 + 2^-8 is the exact midpoint between 1 and 1 + 2^-7: ties to even -> 1.0.
    # Adding 2^-40 puts it above the midpoint; a detour through fp32 would lose that bit.
    enc = lambda x: int(oracle.bf16_encode(np.array([x]))[0])
    assert enc(1.0 + 2.0 ** -8) == 0x3F80
    assert enc(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert enc(1.0 + 3 * 2.0 ** -8) == 0x3F82       # midpoint 1+2^-7 / 1+2^-6 -> even (0x82)
    assert enc(1e39) == 0x7F80 and enc(-1e39) == 0xFF80
    assert enc(math.nan) & 0x7FC0 == 0x7FC0


@pytest.mark.parametrize("bits", [0x0000, 0x3F80, 0xBF80, 0x7F7F, 0x0001, 0x4049])
def test_bf16_decode_is_exact(bits):
    v = oracle.bf16_decode(np.array([bits], np.uint16))[0]
    assert oracle.lib().oracle_bf16_decode(bits) == v
    assert int(oracle.bf16_encode(np.array([v]))[0]) == bits


# --- IEEE binary16 (the table form's "activation dtype" may be float16) ------------------------

def test_f16_decode_every_code_matches_ieee_binary16():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_decode(codes)
    ref = codes.view(np.float16).astype(np.float64)   # numpy's IEEE-754 binary16
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_f16_encode_hand_values():
    enc = lambda x: int(oracle.f16_encode(np.array([x]))[0])
    assert enc(1.0) == 0x3C00 and enc(-2.0) == 0xC000
    assert enc(65504.0) == 0x7BFF                      # largest finite
    assert enc(65519.99) == 0x7BFF                     # below the overflow midpoint
    assert enc(65520.0) == 0x7C00                      # midpoint ties to even = infinity
    assert enc(2.0 ** -24) == 0x0001                   # smallest subnormal
    assert enc(2.0 ** -25) == 0x0000                   # half of it: tie to even (zero)
    assert enc(3 * 2.0 ** -25) == 0x0002               # 1.5 quanta -> 2
    assert enc(2.0 ** -14) == 0x0400                   # smallest normal
    assert enc(1.0 + 2.0 ** -11) == 0x3C00             # tie between 1 and 1+2^-10 -> even
    assert enc(1.0 + 3 * 2.0 ** -11) == 0x3C02         # tie -> even mantissa 2
    assert enc(math.inf) == 0x7C00 and enc(-math.inf) == 0xFC00
    assert enc(-0.0) == 0x8000
    assert np.isnan(oracle.f16_decode(np.array([enc(math.nan)], np.uint16))[0])


def test_f16_encode_matches_numpy_rounding():
    rng = np.random.default_rng(17)
    x = np.concatenate([rng.standard_normal(40000) * s for s in (1e-7, 1e-3, 1.0, 3e3, 6e4)])
    # every midpoint between neighbouring finite codes, and just either side of it
    fin = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (fin[1:] + fin[:-1]) / 2
    x = np.concatenate([x, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf)])
    ours = oracle.f16_encode(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)      # numpy rounds double -> half to nearest even
    np.testing.assert_array_equal(ours, ref)
    # every finite code encodes back to itself
    codes = np.arange(0, 0x7C00, dtype=np.uint16)
    np.testing.assert_array_equal(oracle.f16_encode(oracle.f16_decode(codes)), codes)
