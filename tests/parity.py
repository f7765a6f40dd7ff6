"""Shared helpers for the GPU parity tests: running both sides and the match criteria.

Match criteria (element by element against the fp64 oracle on the same seeded inputs):
  * V copy (bf16 output): bit-exact.
  * bf16 Q/K: |gpu - ref| <= 2^-7 * |ref| + 1e-3, with ref the oracle's unrounded fp64 value.
  * FP8 E4M3 outputs: within one code of the oracle's round-to-nearest-even code (codes compared
    in sign-magnitude order, so +0 and -0 are the same point).
  * float16 Q/K (table form with binary16 activations): |gpu - ref| <= 2^-10 * |ref| + 2^-14.
    One rounding to binary16 costs at most half an ulp (2^-11 relative for normal values); fp32
    arithmetic before it can move a value across one rounding boundary, hence one ulp (2^-10);
    the absolute term is the smallest normal binary16 (subnormal outputs have a fixed quantum).
  * camera prologue outputs (16-bit): |gpu - ref| <= u * |ref| + 2^-16 * max|ref|, u = 2^-7
    (bf16) or 2^-10 (binary16): one ulp of the output format as above, plus the fp32
    accumulation of the 4-term projection and the rotation (a few 2^-24 of the largest
    intermediate, bounded by the tensor's largest magnitude), so that tensors of small
    magnitude (K after k_scale ~ 0.004) are held to the same relative standard; binary16 adds
    its subnormal quantum 2^-24.
  * inflation_sq (fp32): relative 2^-16 (fp32 sums of head_dim squares and one division).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

BF16_REL = 2.0 ** -7
BF16_ABS = 1e-3

# Observed error of every 16-bit and E4M3 comparison made in this process, by label (the label's
# first word is the workload or case name): how many outputs equal the oracle's
# round-to-nearest-even result bit for bit or lie within one unit in the last place (one code,
# for E4M3); the largest such distance among outputs where the relative part of the tolerance
# governs (|ref| >= 2^-3 for bf16, where 2^-7 |ref| >= 1e-3; near zero a few ulps of fp32
# cancellation in the rotation span many tiny 16-bit ulps); and the largest share of its
# tolerance any output uses (err / bound). The pass criterion stays the tolerance above;
# conftest.py prints these figures at the end of a session and writes them as JSON to
# $QKROPE_PARITY_REPORT if set.
OBSERVED: dict[str, dict] = {}


def _ordinal16(bits: np.ndarray) -> np.ndarray:
    """Position of a 16-bit float pattern on the number line, +0 and -0 both at 0."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def record_observed(what: str, gpu_bits: np.ndarray, ref_bits: np.ndarray, ordinal,
                    large: np.ndarray | None = None, tol_used: float = 0.0) -> None:
    """Add one comparison to OBSERVED[what]: ulp distances of the outputs (large: the outputs
    whose max ulp is reported, all if None) and the largest share of tolerance used."""
    g, r = gpu_bits.ravel(), ref_bits.ravel()
    d = np.abs(ordinal(g) - ordinal(r))
    dl = d if large is None else d[large.ravel()]
    e = OBSERVED.setdefault(what, {"n": 0, "bit_equal": 0, "within_1ulp": 0, "max_ulp": 0,
                                   "max_tol_used": 0.0})
    e["n"] += int(d.size)
    e["bit_equal"] += int((d == 0).sum())
    e["within_1ulp"] += int((d <= 1).sum())
    e["max_ulp"] = max(e["max_ulp"], int(dl.max()) if dl.size else 0)
    e["max_tol_used"] = max(e["max_tol_used"], float(tol_used))


def _observe_16(gpu: torch.Tensor, ref: np.ndarray, what: str, tol_used: float,
                large_from: float) -> None:
    keep = ~np.isnan(ref)
    enc = oracle.f16_encode if gpu.dtype == torch.float16 else oracle.bf16_encode
    g = bits16(gpu).reshape(ref.shape)[keep]
    record_observed(what, g, enc(ref[keep]), _ordinal16, np.abs(ref[keep]) >= large_from,
                    tol_used)


def _tol_used(err: np.ndarray, bound: np.ndarray) -> float:
    with np.errstate(invalid="ignore", divide="ignore"):
        f = np.where(bound > 0, err / bound, 0.0)
    f = f[np.isfinite(f)]
    return float(f.max()) if f.size else 0.0


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def codes8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def assert_bf16_close(gpu: torch.Tensor, ref: np.ndarray, what: str) -> None:
    g = to_f64(gpu).reshape(ref.shape)
    err = np.abs(g - ref)
    bound = BF16_REL * np.abs(ref) + BF16_ABS
    _observe_16(gpu, ref, what, _tol_used(err, bound), BF16_ABS / BF16_REL)
    bad = ~(err <= bound)
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        idx = np.unravel_index(i, ref.shape)
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; first at {idx}: "
            f"gpu={g[idx]!r} ref={ref[idx]!r} err={err[idx]:.3g} bound={bound[idx]:.3g}")


F16_REL = 2.0 ** -10
F16_ABS = 2.0 ** -14


def assert_f16_close(gpu: torch.Tensor, ref: np.ndarray, what: str) -> None:
    assert gpu.dtype == torch.float16, f"{what}: expected float16 output, got {gpu.dtype}"
    g = to_f64(gpu).reshape(ref.shape)
    err = np.abs(g - ref)
    bound = F16_REL * np.abs(ref) + F16_ABS
    _observe_16(gpu, ref, what, _tol_used(err, bound), F16_ABS / F16_REL)
    bad = ~(err <= bound)
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        idx = np.unravel_index(i, ref.shape)
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; first at {idx}: "
            f"gpu={g[idx]!r} ref={ref[idx]!r} err={err[idx]:.3g} bound={bound[idx]:.3g}")


def e4m3_ordinal(codes: np.ndarray) -> np.ndarray:
    c = codes.astype(np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def assert_e4m3_within_one(gpu: torch.Tensor, ref_codes: np.ndarray, what: str) -> None:
    g = codes8(gpu).reshape(ref_codes.shape)
    assert not np.any((g & 0x7F) == 0x7F), f"{what}: NaN code in GPU output"
    d = np.abs(e4m3_ordinal(g) - e4m3_ordinal(ref_codes))
    record_observed(what, g, ref_codes, e4m3_ordinal, None, float(d.max()) if d.size else 0.0)
    if (d > 1).any():
        i = np.flatnonzero((d > 1).ravel())[0]
        idx = np.unravel_index(i, ref_codes.shape)
        raise AssertionError(f"{what}: {(d > 1).sum()} codes more than one step away; first at "
                             f"{idx}: gpu=0x{g[idx]:02x} ref=0x{ref_codes[idx]:02x}")


def assert_bits_equal(gpu: torch.Tensor, ref_bits: np.ndarray, what: str) -> None:
    g = bits16(gpu).reshape(ref_bits.shape) if gpu.dtype == torch.bfloat16 else \
        codes8(gpu).reshape(ref_bits.shape)
    if not np.array_equal(g, ref_bits):
        n = int((g != ref_bits).sum())
        raise AssertionError(f"{what}: {n} of {g.size} elements differ (bit-exact required)")


def check_3d_outputs(w, outs, ref, tokens=None) -> None:
    """Compare GPU (q, k, v) of a 3D workload with the oracle's fp64 (q, k, v).

    `tokens` selects flattened token rows of the GPU outputs that `ref` covers (None: all).
    """
    names = ("q", "k", "v")
    for i, (o, r) in enumerate(zip(outs, ref)):
        H = (w.num_heads_q, w.num_heads_k, w.num_heads_v)[i]
        o = o.reshape(w.num_tokens, H, w.head_dim)
        if tokens is not None:
            o = o[torch.as_tensor(tokens, device=o.device)]
        if w.output_fp8:
            scale = w.v_quant_scale if i == 2 else w.output_quant_scale
            codes = oracle.e4m3_encode(r, scale)
            if i == 2:
                # v * v_quant_scale is exact for a power-of-two scale: one correct code
                if float(np.log2(scale)).is_integer():
                    assert_bits_equal(o, codes, f"{w.name} v (e4m3)")
                else:
                    assert_e4m3_within_one(o, codes, f"{w.name} v (e4m3)")
            else:
                assert_e4m3_within_one(o, codes, f"{w.name} {names[i]} (e4m3)")
        elif i == 2:
            assert_bits_equal(o, oracle.bf16_encode(r), f"{w.name} v")
        else:
            assert_bf16_close(o, r, f"{w.name} {names[i]}")


def check_table_outputs(name, q_out, k_out, ref_q, ref_k) -> None:
    assert_bf16_close(q_out, ref_q, f"{name} q")
    assert_bf16_close(k_out, ref_k, f"{name} k")


def assert_cam_close(gpu: torch.Tensor, ref: np.ndarray, what: str) -> None:
    """Camera prologue 16-bit outputs against the oracle's fp64 values (criteria above)."""
    g = to_f64(gpu).reshape(ref.shape)
    rel = 2.0 ** -10 if gpu.dtype == torch.float16 else 2.0 ** -7
    floor = 2.0 ** -16 * (np.abs(ref).max() if ref.size else 0.0)
    if gpu.dtype == torch.float16:
        floor += 2.0 ** -24
    err = np.abs(g - ref)
    bound = rel * np.abs(ref) + floor
    _observe_16(gpu, ref, what, _tol_used(err, bound), floor / rel)
    bad = ~(err <= bound)
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        idx = np.unravel_index(i, ref.shape)
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; first at {idx}: "
            f"gpu={g[idx]!r} ref={ref[idx]!r} err={err[idx]:.3g} bound={bound[idx]:.3g}")


def assert_inflation_close(gpu: torch.Tensor, ref: np.ndarray, what: str) -> None:
    g = to_f64(gpu).reshape(ref.shape)
    err = np.abs(g - ref)
    bound = 2.0 ** -16 * np.abs(ref)
    bad = ~(err <= bound)
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        idx = np.unravel_index(i, ref.shape)
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} values out of tolerance; first at {idx}: "
            f"gpu={g[idx]!r} ref={ref[idx]!r}")
