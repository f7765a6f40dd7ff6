"""Python binding of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module. The HIP product path never does, and this module imports nothing from
the product package.

Inputs are CPU tensors (bf16 / float16 / float32) or numpy arrays (uint16 bf16 bit patterns,
float16, float32, float64 tables); outputs are float64 numpy arrays, unrounded, plus the encoders
that turn them into bf16 or binary16 bits and OCP E4M3 codes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# QKROPE_ORACLE_LIB: load another build of oracle.c instead (the mutation test runs the pins
# against copies with planted mistakes)
LIB_PATH = os.environ.get("QKROPE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
SOURCE = os.path.join(_HERE, "oracle.c")

NORM_MODES = {"none": 0, "per_head": 1, "across_heads": 2}
TABLE_BF16, TABLE_F32, TABLE_F64, TABLE_F16 = 0, 1, 2, 3
ACT_BF16, ACT_F16 = 0, 1


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (portable x86-64, OpenMP; ISO C, so no
    floating-point contraction or reassociation)."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-o", tmp, SOURCE, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.oracle_run_table.argtypes = [P, P, P, P, P, I, D, I64, I, I, I, I, I, I,
                                       I64, I64, I64, P, P]
        L.oracle_run_table.restype = I
        L.oracle_run_table_split.argtypes = [P, P, P, P, I, P, P, I, D, I64, I, I, I, I, I, I,
                                             I64, I64, I64, I64, P, P]
        L.oracle_run_table_split.restype = I
        L.oracle_sumsq_3d.argtypes = [P, I64, I, I, I, I, P]
        L.oracle_sumsq_3d.restype = I
        L.oracle_cam_prep.argtypes = [P, P, P, I, P, P, P, P, D, I64, I64, I, I, I64, I64, I64,
                                      P, P, P, P]
        L.oracle_cam_prep.restype = I
        L.oracle_f16_encode.argtypes = [D]
        L.oracle_f16_encode.restype = ctypes.c_uint16
        L.oracle_f16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_f16_decode.restype = D
        L.oracle_encode_f16_array.argtypes = [P, I64, P]
        L.oracle_encode_f16_array.restype = None
        L.oracle_run_3d.argtypes = [P, P, P, I64, I64, I, I, I, I, I, I, I, I, I, I,
                                    D, D, I, D, D, D, D, I, P, P, P]
        L.oracle_run_3d.restype = I
        L.oracle_bf16_encode.argtypes = [D]
        L.oracle_bf16_encode.restype = ctypes.c_uint16
        L.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_decode.restype = D
        L.oracle_e4m3_encode.argtypes = [D]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = D
        L.oracle_encode_bf16_array.argtypes = [P, I64, P]
        L.oracle_encode_bf16_array.restype = None
        L.oracle_quantize_e4m3_array.argtypes = [P, I64, D, P]
        L.oracle_quantize_e4m3_array.restype = None
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = I
        _lib = L
    return _lib


def num_threads() -> int:
    return lib().oracle_num_threads()


# --- array helpers -----------------------------------------------------------------------------

def _bits16(x) -> np.ndarray:
    """bf16 bit patterns as a C-contiguous uint16 array (accepts torch bf16 or numpy uint16)."""
    if hasattr(x, "detach"):                       # torch tensor
        import torch
        x = x.detach()
        if x.dtype != torch.bfloat16:
            raise TypeError(f"expected a bfloat16 tensor, got {x.dtype}")
        x = x.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError(f"expected uint16 bf16 bits, got {x.dtype}")
    return x


def _act_bits(x):
    """(uint16 bits, activation code) of 16-bit activations: torch bf16 or float16, numpy
    uint16 (bf16 bit patterns) or float16."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach()
        if x.dtype == torch.float16:
            x = x.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
            return np.ascontiguousarray(x), ACT_F16
        return _bits16(x), ACT_BF16
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        return x.view(np.uint16), ACT_F16
    return _bits16(x), ACT_BF16


def _table(x):
    """(array, dtype code) for a rope table: torch bf16/float16/fp32, numpy uint16 (bf16 bits)
    /float16/float32/float64."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().cpu().contiguous()
        if x.dtype == torch.float32:
            return np.ascontiguousarray(x.numpy()), TABLE_F32
        bits, act = _act_bits(x)
        return bits, TABLE_F16 if act == ACT_F16 else TABLE_BF16
    x = np.ascontiguousarray(x)
    if x.dtype == np.float64:
        return x, TABLE_F64
    if x.dtype == np.float32:
        return x, TABLE_F32
    if x.dtype == np.float16:
        return x.view(np.uint16), TABLE_F16
    return _bits16(x), TABLE_BF16


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# --- the two forms -----------------------------------------------------------------------------

def run_table(q, k, q_weight, k_weight, rope_table, eps, *, rotary_dim=None,
              interleaved=False, norm_mode="per_head", sin_table=None):
    """fp64 table form. q [T,Hq,D], k [T,Hk,D] bf16 or float16 (weights alike).

    With sin_table None, rope_table is the pages' packed [T, >=R] = [cos | sin] table. Otherwise
    rope_table is the [T, >=R/2] cosine table and sin_table the matching sine table (the split
    layout). Returns (q_out, k_out) fp64, unrounded."""
    qb, act = _act_bits(q)
    kb, act_k = _act_bits(k)
    if act_k != act:
        raise ValueError("q and k must share the activation dtype")
    if qb.ndim != 3 or kb.ndim != 3:
        raise ValueError("q and k must be [tokens, heads, head_dim]")
    T, Hq, D = qb.shape
    Hk = kb.shape[1]
    tab, tdt = _table(rope_table)
    wq = _act_bits(q_weight)[0] if q_weight is not None else np.zeros(1, np.uint16)
    wk = _act_bits(k_weight)[0] if k_weight is not None else np.zeros(1, np.uint16)
    qo = np.empty((T, Hq, D), np.float64)
    ko = np.empty((T, Hk, D), np.float64)
    if sin_table is None:
        R = tab.shape[1] if rotary_dim is None else rotary_dim
        if act != ACT_BF16:
            # the packed row seen as the split layout: sine columns start R/2 after the cosines
            sin_ptr = ctypes.c_void_p(tab.ctypes.data + (R // 2) * tab.itemsize)
            rc = lib().oracle_run_table_split(_ptr(qb), _ptr(kb), _ptr(wq), _ptr(wk), act,
                                              _ptr(tab), sin_ptr, tdt, float(eps), T, Hq, Hk,
                                              D, R, int(bool(interleaved)),
                                              NORM_MODES[norm_mode], Hq * D, Hk * D,
                                              tab.shape[1], tab.shape[1], _ptr(qo), _ptr(ko))
        else:
            rc = lib().oracle_run_table(_ptr(qb), _ptr(kb), _ptr(wq), _ptr(wk), _ptr(tab), tdt,
                                        float(eps), T, Hq, Hk, D, R, int(bool(interleaved)),
                                        NORM_MODES[norm_mode], Hq * D, Hk * D, tab.shape[1],
                                        _ptr(qo), _ptr(ko))
    else:
        stab, sdt = _table(sin_table)
        if sdt != tdt:
            raise ValueError("cos and sin tables must share a dtype")
        R = 2 * tab.shape[1] if rotary_dim is None else rotary_dim
        rc = lib().oracle_run_table_split(_ptr(qb), _ptr(kb), _ptr(wq), _ptr(wk), act,
                                          _ptr(tab), _ptr(stab), tdt, float(eps), T, Hq, Hk, D,
                                          R, int(bool(interleaved)), NORM_MODES[norm_mode],
                                          Hq * D, Hk * D, tab.shape[1], stab.shape[1],
                                          _ptr(qo), _ptr(ko))
    if rc != 0:
        raise ValueError(f"oracle table form rejected its arguments (code {rc})")
    return qo, ko


def run_3d(qkv, q_weight, k_weight, *, ppf, pph, ppw, num_frame_channels,
           num_height_channels, num_width_channels, num_heads_q, num_heads_k, num_heads_v,
           head_dim, eps=1e-6, base=10000.0, interleave=True, factor=1.0, low=0.0, high=0.0,
           attention_factor=1.0, is_qk_norm=True, token_offset=0):
    """fp64 3D form over rows of packed qkv. Returns (q, k, v) fp64 [T, H, D], unrounded.

    qkv may be [T, row] or [B, S, row]; token_offset is the flattened index of its first row.
    """
    x = _bits16(qkv)
    row = (num_heads_q + num_heads_k + num_heads_v) * head_dim
    x = x.reshape(-1, row)
    T = x.shape[0]
    D = head_dim
    wq = _bits16(q_weight) if q_weight is not None else np.zeros(1, np.uint16)
    wk = _bits16(k_weight) if k_weight is not None else np.zeros(1, np.uint16)
    qo = np.empty((T, num_heads_q, D), np.float64)
    ko = np.empty((T, num_heads_k, D), np.float64)
    vo = np.empty((T, num_heads_v, D), np.float64)
    rc = lib().oracle_run_3d(_ptr(x), _ptr(wq), _ptr(wk), T, int(token_offset), ppf, pph, ppw,
                             num_frame_channels, num_height_channels, num_width_channels,
                             num_heads_q, num_heads_k, num_heads_v, D, float(eps), float(base),
                             int(bool(interleave)), float(factor), float(low), float(high),
                             float(attention_factor), int(bool(is_qk_norm)),
                             _ptr(qo), _ptr(ko), _ptr(vo))
    if rc != 0:
        raise ValueError(f"oracle_run_3d rejected its arguments (code {rc})")
    return qo, ko, vo


def sumsq_3d(qkv, *, num_heads_q, num_heads_k, num_heads_v, head_dim) -> np.ndarray:
    """Per-token sums of squares of the Q and K rows of packed bf16 qkv, fp64 [T, 2]."""
    x = _bits16(qkv)
    row = (num_heads_q + num_heads_k + num_heads_v) * head_dim
    x = x.reshape(-1, row)
    out = np.empty((x.shape[0], 2), np.float64)
    rc = lib().oracle_sumsq_3d(_ptr(x), x.shape[0], num_heads_q, num_heads_k, num_heads_v,
                               head_dim, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_sumsq_3d rejected its arguments (code {rc})")
    return out


def _f32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch
        x = x.detach().cpu()
        if x.dtype != torch.float32:
            raise TypeError(f"expected a float32 tensor, got {x.dtype}")
        x = x.numpy()
    x = np.ascontiguousarray(x)
    if x.dtype != np.float32:
        raise TypeError(f"expected float32, got {x.dtype}")
    return x


def cam_prep(q, k, v, proj_q, proj_kv, rope_cos, rope_sin, k_scale, *, num_heads=None,
             head_dim=None):
    """fp64 camera prologue (UCPE page, cam_prep_func) under the readings in oracle.c.

    q, k, v: [B, N, H, D] bf16 or float16 (or [B, N, S] rows of S >= H*D elements with
    num_heads and head_dim given); proj_q, proj_kv: [B, N, 4, 4] float32; rope_cos, rope_sin:
    [N, D/2] float32. Returns q_out, k_out, v_out fp64 [B, H, D, N] and inflation_sq fp64
    [B, H, N], unrounded."""
    xs = [_act_bits(t) for t in (q, k, v)]
    acts = {a for _, a in xs}
    if len(acts) != 1:
        raise ValueError("q, k and v must share the activation dtype")
    act = acts.pop()
    bits = [b for b, _ in xs]
    if bits[0].ndim == 4:
        B, N, H, D = bits[0].shape
    else:
        B, N = bits[0].shape[:2]
        H, D = int(num_heads), int(head_dim)
    strides = [int(np.prod(b.shape[2:])) for b in bits]
    if any(st < H * D for st in strides) or any(b.shape[:2] != (B, N) for b in bits):
        raise ValueError("q, k, v must be [B, N, H, D] (or rows of at least H*D elements)")
    pq, pkv = _f32(proj_q), _f32(proj_kv)
    tc, ts = _f32(rope_cos), _f32(rope_sin)
    if pq.shape != (B, N, 4, 4) or pkv.shape != (B, N, 4, 4):
        raise ValueError("projections must be [B, N, 4, 4]")
    if tc.shape != (N, D // 2) or ts.shape != (N, D // 2):
        raise ValueError("rope tables must be [N, D/2]")
    outs = [np.empty((B, H, D, N), np.float64) for _ in range(3)]
    infl = np.empty((B, H, N), np.float64)
    rc = lib().oracle_cam_prep(_ptr(bits[0]), _ptr(bits[1]), _ptr(bits[2]), act, _ptr(pq),
                               _ptr(pkv), _ptr(tc), _ptr(ts), float(k_scale), B, N, H, D,
                               strides[0], strides[1], strides[2], _ptr(outs[0]),
                               _ptr(outs[1]), _ptr(outs[2]), _ptr(infl))
    if rc != 0:
        raise ValueError(f"oracle_cam_prep rejected its arguments (code {rc})")
    return outs[0], outs[1], outs[2], infl


def run_3d_workload(w, qkv, q_weight, k_weight, token_offset=0):
    """run_3d with the parameters of a 3D workload description (any object with those fields)."""
    return run_3d(qkv, q_weight, k_weight, ppf=w.ppf, pph=w.pph, ppw=w.ppw,
                  num_frame_channels=w.num_frame_channels,
                  num_height_channels=w.num_height_channels,
                  num_width_channels=w.num_width_channels, num_heads_q=w.num_heads_q,
                  num_heads_k=w.num_heads_k, num_heads_v=w.num_heads_v, head_dim=w.head_dim,
                  eps=w.eps, base=w.base, interleave=w.interleave, factor=w.factor, low=w.low,
                  high=w.high, attention_factor=w.attention_factor, is_qk_norm=w.is_qk_norm,
                  token_offset=token_offset)


# --- encoders ----------------------------------------------------------------------------------

def bf16_encode(x) -> np.ndarray:
    """Round-to-nearest-even bf16 bit patterns of an fp64 array."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, np.uint16)
    lib().oracle_encode_bf16_array(_ptr(a), a.size, _ptr(out))
    return out


def bf16_decode(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_encode(x) -> np.ndarray:
    """Round-to-nearest-even IEEE binary16 bit patterns (uint16) of an fp64 array."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, np.uint16)
    lib().oracle_encode_f16_array(_ptr(a), a.size, _ptr(out))
    return out


def f16_decode(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    f = lib().oracle_f16_decode
    table = np.array([f(i) for i in range(65536)], dtype=np.float64)
    return table[b]


def e4m3_encode(x, scale: float = 1.0) -> np.ndarray:
    """OCP E4M3 codes of x*scale (RNE, saturating to +-448, NaN kept)."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, np.uint8)
    lib().oracle_quantize_e4m3_array(_ptr(a), a.size, float(scale), _ptr(out))
    return out


def e4m3_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    f = lib().oracle_e4m3_decode
    table = np.array([f(i) for i in range(256)], dtype=np.float64)
    return table[c]
