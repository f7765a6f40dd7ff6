"""Fused QK-RMSNorm + RoPE (+ V) attention prologue for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in include/qkrope.h (libqkrope.so, built by build.py). The
binding only marshals arguments: every step of the computation runs in the library's HIP
kernels. PyTorch provides device memory and the current stream.

Entry points, with the names of the C ABI:
  qkrope_create / qkrope_destroy / qkrope_run_table / qkrope_run_3d
  qkrope_run_table_ex (split cos/sin tables, float16 activations, E4M3 outputs)
  qkrope_sumsq_3d / qkrope_run_3d_sharded (sequence- and head-sharded 3D form)
  qkrope_min_tokens (fused-vs-eager threshold, QKROPE_FUSED_MIN_TOKENS)
  qkrope_cam_prep (camera prologue of the SANA-WM UCPE branch)
and the page-shaped conveniences that allocate outputs:
  fused_qk_norm_rope      -- vLLM-Omni "vllm_omni.diffusion.layers.fused_qk_norm_rope"
  fused_qk_rmsnorm_rope   -- FlashInfer "flashinfer.norm.fused_qk_rmsnorm_rope"
  cam_prep_func           -- vLLM-Omni "vllm_omni.diffusion.models.sana_wm.ucpe"

There is no fallback: if the library is missing or the device is not gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch  # imported before the library so both share torch's HIP runtime


LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqkrope.so")

QKROPE_OK, QKROPE_ERR_INVALID, QKROPE_ERR_UNSUPPORTED, QKROPE_ERR_DEVICE, QKROPE_ERR_ALLOC = range(5)
QKROPE_DTYPE_BF16, QKROPE_DTYPE_F32, QKROPE_DTYPE_F16, QKROPE_DTYPE_E4M3 = 0, 1, 2, 3
QKROPE_TABLE_BF16, QKROPE_TABLE_F32 = QKROPE_DTYPE_BF16, QKROPE_DTYPE_F32
NORM_MODES = {"none": 0, "per_head": 1, "across_heads": 2}

_lock = threading.Lock()
_lib = None
_handles: dict[int, int] = {}


class QkropeError(RuntimeError):
    """A device-side failure reported by the library (status QKROPE_ERR_DEVICE / _ALLOC)."""


def _hip_runtimes_loaded() -> set[str]:
    with open("/proc/self/maps") as f:
        return {l.split()[-1] for l in f if "libamdhip64" in l}


def lib() -> ctypes.CDLL:
    """Load libqkrope.so (once). Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'` "
                               "or `python qk_rmsnorm_rope_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.qkrope_create.argtypes = [I, ctypes.POINTER(P)]
        L.qkrope_create.restype = I
        L.qkrope_destroy.argtypes = [P]
        L.qkrope_destroy.restype = I
        L.qkrope_status_str.argtypes = [I]
        L.qkrope_status_str.restype = ctypes.c_char_p
        L.qkrope_last_error.argtypes = []
        L.qkrope_last_error.restype = ctypes.c_char_p
        L.qkrope_run_table.argtypes = [P, P, P, P, P, P, I, D, I64, I, I, I, I, I, I,
                                       I64, I64, I64, P, P, I64, I64, P]
        L.qkrope_run_table.restype = I
        L.qkrope_run_3d.argtypes = [P, P, P, P, I64, I, I, I, I, I, I, I, I, I, I,
                                    D, D, I, D, D, D, D, I, I, D, D, P, P, P, P]
        L.qkrope_run_3d.restype = I
        L.qkrope_min_tokens.argtypes = [I64, ctypes.POINTER(I64)]
        L.qkrope_min_tokens.restype = I
        L.qkrope_run_table_ex.argtypes = [P, P, P, P, P, P, P, I, I, I, D, D, I64, I, I, I, I,
                                          I, I, I64, I64, I64, I64, P, P, I64, I64, P]
        L.qkrope_run_table_ex.restype = I
        L.qkrope_sumsq_3d.argtypes = [P, P, I64, I, I, I, I, P, P]
        L.qkrope_sumsq_3d.restype = I
        L.qkrope_run_3d_sharded.argtypes = [P, P, P, P, I64, I64, P, I64, I64, I, I, I, I, I, I,
                                            I, I, I, I, D, D, I, D, D, D, D, I, I, D, D,
                                            P, P, P, P]
        L.qkrope_run_3d_sharded.restype = I
        L.qkrope_cam_prep.argtypes = [P, P, P, P, I, P, P, P, P, ctypes.c_float, I64, I64, I, I,
                                      I64, I64, I64, P, P, P, I64, P, P]
        L.qkrope_cam_prep.restype = I
        runtimes = _hip_runtimes_loaded()
        if len(runtimes) > 1:
            raise RuntimeError(f"two HIP runtimes are loaded ({sorted(runtimes)}); "
                               "libqkrope.so must share torch's")
        _lib = L
        return L


def _check(status: int, what: str) -> None:
    if status == QKROPE_OK:
        return
    L = lib()
    msg = f"{what}: {L.qkrope_status_str(status).decode()}: {L.qkrope_last_error().decode()}"
    if status in (QKROPE_ERR_INVALID, QKROPE_ERR_UNSUPPORTED):
        raise ValueError(msg)
    raise QkropeError(msg)


# --- the C entry points ------------------------------------------------------------------------

def qkrope_create(device: int = 0) -> int:
    """Create a library handle for HIP device `device`; returns the opaque handle."""
    h = ctypes.c_void_p()
    _check(lib().qkrope_create(int(device), ctypes.byref(h)), "qkrope_create")
    return h.value


def qkrope_destroy(handle) -> None:
    _check(lib().qkrope_destroy(handle), "qkrope_destroy")


def qkrope_min_tokens(default: int) -> int:
    """Token count below which a consumer should keep its eager chain: `default` unless the
    QKROPE_FUSED_MIN_TOKENS environment variable overrides it (read at every call; 0 = always
    fuse; unset or blank = default; anything but a non-negative integer raises ValueError)."""
    out = ctypes.c_int64()
    _check(lib().qkrope_min_tokens(int(default), ctypes.byref(out)), "qkrope_min_tokens")
    return out.value


def fused_qk_norm_rope_min_tokens(default: int) -> int:
    """vLLM-Omni's fused_qk_norm_rope_min_tokens signature over qkrope_min_tokens."""
    return qkrope_min_tokens(default)


def _handle_for(device: torch.device) -> int:
    idx = device.index if device.index is not None else torch.cuda.current_device()
    with _lock:
        h = _handles.get(idx)
    if h is None:
        h = qkrope_create(idx)
        with _lock:
            _handles.setdefault(idx, h)
            h = _handles[idx]
    return h


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _same_device(device: torch.device, **tensors) -> None:
    """Every given tensor (None skipped) must be a GPU tensor on `device`: the library reads and
    writes through the raw pointers, so a host tensor or another GPU's must be refused here."""
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {device}")
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device != device):
            raise ValueError(f"{name} must be a GPU tensor on {device}, got {t.device}")


_C_INT_MIN, _C_INT_MAX = -(1 << 31), (1 << 31) - 1


def _c_ints(**values) -> None:
    """Arguments the C ABI takes as `int`: ctypes would truncate a larger value to its low 32
    bits without a word (2**32 + 20 passed as 20), so each must fit before the call."""
    for name, v in values.items():
        if not _C_INT_MIN <= v <= _C_INT_MAX:
            raise ValueError(f"{name} = {v} does not fit the C ABI's 32-bit int")


def _check_weight(w, need: int, dtype, name: str) -> None:
    """A norm weight: contiguous, of `dtype`, holding at least the `need` elements the kernels
    read (the C ABI takes a bare pointer, so its length is checked here). A region that reads
    none (no heads) may pass None."""
    if w is None and need == 0:
        return
    if w is None or w.dtype != dtype or not w.is_contiguous() or w.numel() < need:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of at least {need} elements")


def _weight_elems(norm_mode: str, heads: int, head_dim: int) -> int:
    """Elements of one region's norm weight that a call reads: [head_dim] per head, [heads *
    head_dim] across heads, none for a region without heads or without norm."""
    if norm_mode == "none" or heads == 0:
        return 0
    return heads * head_dim if norm_mode == "across_heads" else head_dim


def _rows(t: torch.Tensor, heads: int, head_dim: int, name: str) -> int:
    """Token stride (elements) of a [T, H, D] (or [T, H*D]) view with contiguous heads/dims."""
    if t.dim() == 3:
        ok = t.shape[1] == heads and t.shape[2] == head_dim and \
            (t.shape[1] <= 1 or t.stride(1) == head_dim) and (t.shape[2] <= 1 or t.stride(2) == 1)
    elif t.dim() == 2:
        ok = t.shape[1] == heads * head_dim and (t.shape[1] <= 1 or t.stride(1) == 1)
    else:
        ok = False
    if not ok:
        raise ValueError(f"{name} must be [tokens, heads, head_dim] with contiguous heads and dims")
    return t.stride(0) if t.shape[0] > 1 else heads * head_dim


def qkrope_run_table(q, k, q_weight, k_weight, rope_table, eps, *, q_out, k_out,
                     head_dim=None, rotary_dim=None, interleaved=False, norm_mode="per_head",
                     stream=None) -> None:
    """Table form into caller-provided outputs (q_out may be q, k_out may be k)."""
    for name, t in (("q", q), ("k", k), ("q_out", q_out), ("k_out", k_out)):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise ValueError(f"{name} must be a bfloat16 GPU tensor")
    D = head_dim if head_dim is not None else q.shape[-1]
    Hq = q.shape[1] if q.dim() == 3 else q.shape[1] // D
    Hk = k.shape[1] if k.dim() == 3 else k.shape[1] // D
    T = q.shape[0]
    if k.shape[0] != T or q_out.shape[0] != T or k_out.shape[0] != T:
        raise ValueError("q, k and outputs must have the same number of tokens")
    R = rotary_dim if rotary_dim is not None else rope_table.shape[-1]
    if rope_table.dtype == torch.float32:
        tdt = QKROPE_TABLE_F32
    elif rope_table.dtype == torch.bfloat16:
        tdt = QKROPE_TABLE_BF16
    else:
        raise ValueError("rope_table must be float32 or bfloat16")
    if rope_table.dim() != 2 or rope_table.shape[0] != T or rope_table.shape[1] < R or \
            (R > 0 and rope_table.stride(1) != 1) or not rope_table.is_cuda:
        raise ValueError("rope_table must be a GPU [tokens, >= rotary_dim] tensor whose "
                         "columns are contiguous (unit stride along the last dim)")
    ts = rope_table.stride(0) if T > 1 else rope_table.shape[1]
    if norm_mode not in NORM_MODES:
        raise ValueError(f"norm_mode must be one of {sorted(NORM_MODES)}")
    if norm_mode != "none":
        for name, w, H in (("q_weight", q_weight, Hq), ("k_weight", k_weight, Hk)):
            _check_weight(w, _weight_elems(norm_mode, H, D), torch.bfloat16, name)
    wq, wk = (q_weight, k_weight) if norm_mode != "none" else (None, None)
    _same_device(q.device, k=k, q_out=q_out, k_out=k_out, rope_table=rope_table, q_weight=wq,
                 k_weight=wk)
    s = lib().qkrope_run_table(
        _handle_for(q.device), _ptr(q), _ptr(k), _ptr(q_weight), _ptr(k_weight), _ptr(rope_table),
        tdt, float(eps), T, Hq, Hk, D, R, int(bool(interleaved)), NORM_MODES[norm_mode],
        _rows(q, Hq, D, "q"), _rows(k, Hk, D, "k"), ts, _ptr(q_out), _ptr(k_out),
        _rows(q_out, Hq, D, "q_out"), _rows(k_out, Hk, D, "k_out"), _stream(q.device, stream))
    _check(s, "qkrope_run_table")


_DTYPE_CODES = {torch.bfloat16: QKROPE_DTYPE_BF16, torch.float16: QKROPE_DTYPE_F16,
                torch.float32: QKROPE_DTYPE_F32, torch.float8_e4m3fn: QKROPE_DTYPE_E4M3}


def _table_cols(t, T, cols, name) -> int:
    """Token stride of a GPU [tokens, >= cols] table with unit column stride."""
    if t.dim() != 2 or t.shape[0] != T or t.shape[1] < cols or not t.is_cuda or \
            (cols > 0 and t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a GPU [tokens, >= {cols}] tensor whose columns are "
                         "contiguous")
    return t.stride(0) if T > 1 else t.shape[1]


def qkrope_run_table_ex(q, k, q_weight, k_weight, cos_table, sin_table, eps, *, q_out, k_out,
                        head_dim=None, rotary_dim=None, interleaved=False, norm_mode="per_head",
                        out_scale=1.0, stream=None) -> None:
    """Table form with separate [tokens, rotary_dim/2] cos and sin tables, bfloat16 or float16
    activations (weights alike), and outputs in the activation dtype or float8_e4m3fn (codes of
    y * out_scale). Formats are taken from the tensors' dtypes."""
    act = _DTYPE_CODES.get(q.dtype)
    if act not in (QKROPE_DTYPE_BF16, QKROPE_DTYPE_F16) or k.dtype != q.dtype:
        raise ValueError("q and k must both be bfloat16 or both float16")
    out = _DTYPE_CODES.get(q_out.dtype)
    if out not in (act, QKROPE_DTYPE_E4M3) or k_out.dtype != q_out.dtype:
        raise ValueError("q_out and k_out must have q's dtype or float8_e4m3fn")
    tdt = _DTYPE_CODES.get(cos_table.dtype)
    if tdt not in (QKROPE_DTYPE_F32, act) or sin_table.dtype != cos_table.dtype:
        raise ValueError("cos and sin tables must both be float32 or both the activation dtype")
    for name, t in (("q", q), ("k", k), ("q_out", q_out), ("k_out", k_out)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    D = head_dim if head_dim is not None else q.shape[-1]
    Hq = q.shape[1] if q.dim() == 3 else q.shape[1] // D
    Hk = k.shape[1] if k.dim() == 3 else k.shape[1] // D
    T = q.shape[0]
    if k.shape[0] != T or q_out.shape[0] != T or k_out.shape[0] != T:
        raise ValueError("q, k and outputs must have the same number of tokens")
    R = rotary_dim if rotary_dim is not None else 2 * cos_table.shape[-1]
    cs = _table_cols(cos_table, T, R // 2, "cos_table")
    ss = _table_cols(sin_table, T, R // 2, "sin_table")
    if norm_mode not in NORM_MODES:
        raise ValueError(f"norm_mode must be one of {sorted(NORM_MODES)}")
    if norm_mode != "none":
        for name, w, H in (("q_weight", q_weight, Hq), ("k_weight", k_weight, Hk)):
            _check_weight(w, _weight_elems(norm_mode, H, D), q.dtype, name)
    wq, wk = (q_weight, k_weight) if norm_mode != "none" else (None, None)
    _same_device(q.device, k=k, q_out=q_out, k_out=k_out, cos_table=cos_table,
                 sin_table=sin_table, q_weight=wq, k_weight=wk)
    s = lib().qkrope_run_table_ex(
        _handle_for(q.device), _ptr(q), _ptr(k), _ptr(q_weight), _ptr(k_weight),
        _ptr(cos_table), _ptr(sin_table), tdt, act, out, float(out_scale), float(eps), T, Hq, Hk,
        D, R, int(bool(interleaved)), NORM_MODES[norm_mode], _rows(q, Hq, D, "q"),
        _rows(k, Hk, D, "k"), cs, ss, _ptr(q_out), _ptr(k_out), _rows(q_out, Hq, D, "q_out"),
        _rows(k_out, Hk, D, "k_out"), _stream(q.device, stream))
    _check(s, "qkrope_run_table_ex")


def qkrope_sumsq_3d(qkv, *, num_heads_q, num_heads_k, num_heads_v, head_dim, out=None,
                    stream=None) -> torch.Tensor:
    """Per-token fp32 sums of squares of the Q and K rows of packed bf16 qkv: [tokens, 2]."""
    if qkv.dtype != torch.bfloat16 or not qkv.is_cuda or not qkv.is_contiguous():
        raise ValueError("qkv must be a contiguous bfloat16 GPU tensor")
    row = (num_heads_q + num_heads_k + num_heads_v) * head_dim
    if qkv.shape[-1] != row:
        raise ValueError(f"qkv rows must hold {row} elements")
    T = qkv.numel() // row
    if out is None:
        out = torch.empty((T, 2), dtype=torch.float32, device=qkv.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or out.numel() != 2 * T:
        raise ValueError("out must be a contiguous float32 [tokens, 2] tensor")
    _same_device(qkv.device, out=out)
    s = lib().qkrope_sumsq_3d(_handle_for(qkv.device), _ptr(qkv), T, num_heads_q, num_heads_k,
                              num_heads_v, head_dim, _ptr(out), _stream(qkv.device, stream))
    _check(s, "qkrope_sumsq_3d")
    return out


def qkrope_run_3d_sharded(qkv, q_weight, k_weight, *, token_offset=0, sumsq=None,
                          norm_elems_q=0, norm_elems_k=0, ppf, pph, ppw, num_frame_channels,
                          num_height_channels, num_width_channels, num_heads_q, num_heads_k,
                          num_heads_v, head_dim, q_out, k_out, v_out, eps=1e-6, base=10000.0,
                          interleave=True, factor=1.0, low=0.0, high=0.0, attention_factor=1.0,
                          is_qk_norm=True, output_fp8=False, output_quant_scale=1.0,
                          v_quant_scale=1.0, stream=None) -> None:
    """3D form on one shard: tokens from global index token_offset on, and (with sumsq, a
    float32 [tokens, 2] tensor of sums over every head) the across-heads norm of the whole
    row."""
    _c_ints(ppf=ppf, pph=pph, ppw=ppw, num_frame_channels=num_frame_channels,
            num_height_channels=num_height_channels, num_width_channels=num_width_channels,
            num_heads_q=num_heads_q, num_heads_k=num_heads_k, num_heads_v=num_heads_v,
            head_dim=head_dim)
    if qkv.dtype != torch.bfloat16 or not qkv.is_cuda or not qkv.is_contiguous():
        raise ValueError("qkv must be a contiguous bfloat16 GPU tensor")
    row = (num_heads_q + num_heads_k + num_heads_v) * head_dim
    if qkv.shape[-1] != row:
        raise ValueError(f"qkv rows must hold {row} elements")
    T = qkv.numel() // row
    odt = torch.float8_e4m3fn if output_fp8 else torch.bfloat16
    for name, o, H in (("q_out", q_out, num_heads_q), ("k_out", k_out, num_heads_k),
                       ("v_out", v_out, num_heads_v)):
        if o.dtype != odt or not o.is_contiguous() or o.numel() != T * H * head_dim or not o.is_cuda:
            raise ValueError(f"{name} must be a contiguous {odt} GPU tensor of {T}x{H}x{head_dim}")
    if sumsq is not None and (sumsq.dtype != torch.float32 or not sumsq.is_contiguous() or
                              sumsq.numel() != 2 * T or not sumsq.is_cuda):
        raise ValueError("sumsq must be a contiguous float32 GPU tensor [tokens, 2]")
    _same_device(qkv.device, sumsq=sumsq)
    if is_qk_norm:
        for name, w, H in (("q_weight", q_weight, num_heads_q), ("k_weight", k_weight, num_heads_k)):
            _check_weight(w, _weight_elems("across_heads", H, head_dim), torch.bfloat16, name)
    _same_device(qkv.device, q_out=q_out, k_out=k_out, v_out=v_out,
                 q_weight=q_weight if is_qk_norm else None,
                 k_weight=k_weight if is_qk_norm else None)
    s = lib().qkrope_run_3d_sharded(
        _handle_for(qkv.device), _ptr(qkv), _ptr(q_weight) if is_qk_norm else None,
        _ptr(k_weight) if is_qk_norm else None, T, int(token_offset), _ptr(sumsq),
        int(norm_elems_q), int(norm_elems_k), ppf, pph, ppw, num_frame_channels,
        num_height_channels, num_width_channels, num_heads_q, num_heads_k, num_heads_v, head_dim,
        float(eps), float(base), int(bool(interleave)), float(factor), float(low), float(high),
        float(attention_factor), int(bool(is_qk_norm)), int(bool(output_fp8)),
        float(output_quant_scale), float(v_quant_scale), _ptr(q_out), _ptr(k_out), _ptr(v_out),
        _stream(qkv.device, stream))
    _check(s, "qkrope_run_3d_sharded")


def qkrope_run_3d(qkv, q_weight, k_weight, *, ppf, pph, ppw, num_frame_channels,
                  num_height_channels, num_width_channels, num_heads_q, num_heads_k,
                  num_heads_v, head_dim, q_out, k_out, v_out, eps=1e-6, base=10000.0,
                  interleave=True, factor=1.0, low=0.0, high=0.0, attention_factor=1.0,
                  is_qk_norm=True, output_fp8=False, output_quant_scale=1.0, v_quant_scale=1.0,
                  stream=None) -> None:
    """3D form into caller-provided contiguous outputs. qkv is [tokens, row] with tokens a
    multiple of ppf*pph*ppw, or [batch, seq_len, row] with seq_len == ppf*pph*ppw (FlashInfer's
    parameter list: seq_len = ppf * pph * ppw)."""
    _c_ints(ppf=ppf, pph=pph, ppw=ppw, num_frame_channels=num_frame_channels,
            num_height_channels=num_height_channels, num_width_channels=num_width_channels,
            num_heads_q=num_heads_q, num_heads_k=num_heads_k, num_heads_v=num_heads_v,
            head_dim=head_dim)
    row = (num_heads_q + num_heads_k + num_heads_v) * head_dim
    if qkv.dim() not in (2, 3) or qkv.shape[-1] != row:
        raise ValueError(f"qkv must be [tokens, {row}] or [batch, seq_len, {row}]")
    if qkv.dim() == 3 and qkv.shape[1] != ppf * pph * ppw:
        raise ValueError(f"a [batch, seq_len, row] qkv needs seq_len == ppf*pph*ppw = "
                         f"{ppf * pph * ppw}, got {qkv.shape[1]}")
    if qkv.dtype != torch.bfloat16 or not qkv.is_cuda or not qkv.is_contiguous():
        raise ValueError("qkv must be a contiguous bfloat16 GPU tensor")
    T = qkv.numel() // row
    odt = torch.float8_e4m3fn if output_fp8 else torch.bfloat16
    for name, o, H in (("q_out", q_out, num_heads_q), ("k_out", k_out, num_heads_k),
                       ("v_out", v_out, num_heads_v)):
        if o.dtype != odt or not o.is_contiguous() or o.numel() != T * H * head_dim or not o.is_cuda:
            raise ValueError(f"{name} must be a contiguous {odt} GPU tensor of {T}x{H}x{head_dim}")
    if is_qk_norm:
        for name, w, H in (("q_weight", q_weight, num_heads_q), ("k_weight", k_weight, num_heads_k)):
            _check_weight(w, _weight_elems("across_heads", H, head_dim), torch.bfloat16, name)
    _same_device(qkv.device, q_out=q_out, k_out=k_out, v_out=v_out,
                 q_weight=q_weight if is_qk_norm else None,
                 k_weight=k_weight if is_qk_norm else None)
    s = lib().qkrope_run_3d(
        _handle_for(qkv.device), _ptr(qkv), _ptr(q_weight) if is_qk_norm else None,
        _ptr(k_weight) if is_qk_norm else None, T, ppf, pph, ppw, num_frame_channels,
        num_height_channels, num_width_channels, num_heads_q, num_heads_k, num_heads_v, head_dim,
        float(eps), float(base), int(bool(interleave)), float(factor), float(low), float(high),
        float(attention_factor), int(bool(is_qk_norm)), int(bool(output_fp8)),
        float(output_quant_scale), float(v_quant_scale), _ptr(q_out), _ptr(k_out), _ptr(v_out),
        _stream(qkv.device, stream))
    _check(s, "qkrope_run_3d")


# --- the pages' Python signatures --------------------------------------------------------------

# The page signatures are called once per attention site and step, so their host cost matters:
# they are marshalled in C++ (_qkrope_native, built next to libqkrope.so) with the same checks
# and messages as the functions above, then make one call into the same C ABI.
_native_mod = None


def native():
    """The C++ marshaller of the page signatures (loaded once, after libqkrope.so)."""
    global _native_mod
    if _native_mod is None:
        lib()
        try:
            from . import _qkrope_native
        except ImportError as e:
            raise RuntimeError("qk_rmsnorm_rope_amd/_qkrope_native is missing or fails to load "
                               f"({e}): build it with `python qk_rmsnorm_rope_amd/build.py`") from e
        _native_mod = _qkrope_native
    return _native_mod


def _device_error(e: RuntimeError) -> RuntimeError:
    """A library status from the marshaller becomes QkropeError; other errors pass unchanged."""
    return QkropeError(str(e)) if str(e).startswith("qkrope_") else e


def fused_qk_norm_rope(q, k, q_weight, k_weight, rope_table, eps, *, head_dim=None,
                       rotary_dim=None, interleaved=False):
    """Q/K RMSNorm (per head, [head_dim] weights) then RoPE from a [tokens, rotary_dim] table.

    Signature of vLLM-Omni's fused_qk_norm_rope. q/k are bfloat16 or float16; the table is
    float32 or q's dtype. Returns new (q, k) with the inputs' shapes.
    """
    try:
        return (_native_mod or native()).table(
            q, k, q_weight, k_weight, rope_table, float(eps),
            None if head_dim is None else int(head_dim),
            None if rotary_dim is None else int(rotary_dim), bool(interleaved))
    except RuntimeError as e:
        raise _device_error(e) from None


def fused_qk_rmsnorm_rope(qkv, q_weight, k_weight, *, ppf, pph, ppw, num_frame_channels,
                          num_height_channels, num_width_channels, num_heads_q, num_heads_k,
                          num_heads_v, head_dim, eps=1e-6, base=10000.0, interleave=True,
                          factor=1.0, low=0.0, high=0.0, attention_factor=1.0, is_qk_norm=True,
                          output_fp8=False, output_quant_scale=1.0, v_quant_scale=1.0,
                          q_out=None, k_out=None, v_out=None):
    """Across-heads QK RMSNorm + 3D RoPE + V copy (+ FP8), FlashInfer's signature.

    Returns (q_out, k_out, v_out), each [B, S, H, D] for a 3D qkv or [T, H, D] for a 2D one;
    pre-allocated outputs are used when given (destination-passing style). qkv is
    [tokens, row] with tokens a multiple of ppf*pph*ppw, or [batch, seq_len, row] with
    seq_len == ppf*pph*ppw.
    """
    try:
        return (_native_mod or native()).rope3d(
            qkv, q_weight, k_weight, int(ppf), int(pph), int(ppw), int(num_frame_channels),
            int(num_height_channels), int(num_width_channels), int(num_heads_q), int(num_heads_k),
            int(num_heads_v), int(head_dim), float(eps), float(base), bool(interleave),
            float(factor), float(low), float(high), float(attention_factor), bool(is_qk_norm),
            bool(output_fp8), float(output_quant_scale), float(v_quant_scale), q_out, k_out,
            v_out)
    except RuntimeError as e:
        raise _device_error(e) from None


class Prepared3D:
    """Arguments of one qkrope_run_3d call marshalled once, for launching repeatedly with no
    per-call Python work beyond the C call (the tensors must stay alive and unmoved)."""

    def __init__(self, w, qkv, q_weight, k_weight, q_out, k_out, v_out, stream=None):
        # validate once through the regular path (this also launches once)
        qkrope_run_3d(qkv, q_weight, k_weight, ppf=w.ppf, pph=w.pph, ppw=w.ppw,
                      num_frame_channels=w.num_frame_channels,
                      num_height_channels=w.num_height_channels,
                      num_width_channels=w.num_width_channels, num_heads_q=w.num_heads_q,
                      num_heads_k=w.num_heads_k, num_heads_v=w.num_heads_v,
                      head_dim=w.head_dim, q_out=q_out, k_out=k_out, v_out=v_out, eps=w.eps,
                      base=w.base, interleave=w.interleave, factor=w.factor, low=w.low,
                      high=w.high, attention_factor=w.attention_factor,
                      is_qk_norm=w.is_qk_norm, output_fp8=w.output_fp8,
                      output_quant_scale=w.output_quant_scale,
                      v_quant_scale=w.v_quant_scale, stream=stream)
        self._fn = lib().qkrope_run_3d
        self._args = (
            _handle_for(qkv.device), _ptr(qkv), _ptr(q_weight) if w.is_qk_norm else None,
            _ptr(k_weight) if w.is_qk_norm else None, qkv.numel() // w.row_elems, w.ppf, w.pph,
            w.ppw, w.num_frame_channels, w.num_height_channels, w.num_width_channels,
            w.num_heads_q, w.num_heads_k, w.num_heads_v, w.head_dim, float(w.eps),
            float(w.base), int(w.interleave), float(w.factor), float(w.low), float(w.high),
            float(w.attention_factor), int(w.is_qk_norm), int(w.output_fp8),
            float(w.output_quant_scale), float(w.v_quant_scale), _ptr(q_out), _ptr(k_out),
            _ptr(v_out), _stream(qkv.device, stream))
        self._keep = (qkv, q_weight, k_weight, q_out, k_out, v_out)

    def __call__(self) -> None:
        s = self._fn(*self._args)
        if s != QKROPE_OK:
            _check(s, "qkrope_run_3d")


class PreparedTable:
    """Arguments of one table-form call marshalled once (see Prepared3D): qkrope_run_table for
    bf16 in and out with a packed table, qkrope_run_table_ex otherwise (float16 activations or
    E4M3 outputs; the packed table is passed as its cos and sin column views)."""

    def __init__(self, q, k, q_weight, k_weight, rope_table, eps, *, q_out, k_out,
                 head_dim=None, rotary_dim=None, interleaved=False, norm_mode="per_head",
                 out_scale=1.0, stream=None):
        D = head_dim if head_dim is not None else q.shape[-1]
        Hq = q.shape[1] if q.dim() == 3 else q.shape[1] // D
        Hk = k.shape[1] if k.dim() == 3 else k.shape[1] // D
        T = q.shape[0]
        R = rotary_dim if rotary_dim is not None else rope_table.shape[-1]
        common = dict(head_dim=D, rotary_dim=R, interleaved=interleaved, norm_mode=norm_mode,
                      stream=stream)
        ts = rope_table.stride(0) if T > 1 else rope_table.shape[1]
        strides = (_rows(q, Hq, D, "q"), _rows(k, Hk, D, "k"))
        out_strides = (_rows(q_out, Hq, D, "q_out"), _rows(k_out, Hk, D, "k_out"))
        h, st = _handle_for(q.device), _stream(q.device, stream)
        if q.dtype == torch.bfloat16 and q_out.dtype == torch.bfloat16:
            qkrope_run_table(q, k, q_weight, k_weight, rope_table, eps, q_out=q_out, k_out=k_out,
                             **common)
            tdt = QKROPE_TABLE_F32 if rope_table.dtype == torch.float32 else QKROPE_TABLE_BF16
            self._fn, self._name = lib().qkrope_run_table, "qkrope_run_table"
            self._args = (h, _ptr(q), _ptr(k), _ptr(q_weight), _ptr(k_weight), _ptr(rope_table),
                          tdt, float(eps), T, Hq, Hk, D, R, int(bool(interleaved)),
                          NORM_MODES[norm_mode], *strides, ts, _ptr(q_out), _ptr(k_out),
                          *out_strides, st)
        else:
            cos_t, sin_t = rope_table[:, : R // 2], rope_table[:, R // 2: R]
            qkrope_run_table_ex(q, k, q_weight, k_weight, cos_t, sin_t, eps, q_out=q_out,
                                k_out=k_out, out_scale=out_scale, **common)
            self._fn, self._name = lib().qkrope_run_table_ex, "qkrope_run_table_ex"
            self._args = (h, _ptr(q), _ptr(k), _ptr(q_weight), _ptr(k_weight), _ptr(cos_t),
                          _ptr(sin_t), _DTYPE_CODES[rope_table.dtype], _DTYPE_CODES[q.dtype],
                          _DTYPE_CODES[q_out.dtype], float(out_scale), float(eps), T, Hq, Hk, D,
                          R, int(bool(interleaved)), NORM_MODES[norm_mode], *strides, ts, ts,
                          _ptr(q_out), _ptr(k_out), *out_strides, st)
        self._keep = (q, k, q_weight, k_weight, rope_table, q_out, k_out)

    def __call__(self) -> None:
        s = self._fn(*self._args)
        if s != QKROPE_OK:
            _check(s, self._name)


class PreparedSharded3D:
    """One rank's step of a head-sharded 3D run, marshalled once: qkrope_sumsq_3d into `sumsq`,
    then qkrope_run_3d_sharded normalising with `sumsq_total` over `norm_elems_*` elements.
    Between the two a multi-rank caller all-reduces sumsq into sumsq_total; with one rank they
    may be the same tensor. Calling the object runs both; .sumsq() and .apply() run one each."""

    def __init__(self, w, qkv, q_weight, k_weight, q_out, k_out, v_out, sumsq, sumsq_total,
                 token_offset=0, stream=None):
        Hq, Hk, Hv, D = w.num_heads_q, w.num_heads_k, w.num_heads_v, w.head_dim
        T = qkv.numel() // w.row_elems
        ne_q, ne_k = Hq * D * w.head_shards, Hk * D * w.head_shards
        qkrope_sumsq_3d(qkv, num_heads_q=Hq, num_heads_k=Hk, num_heads_v=Hv, head_dim=D,
                        out=sumsq, stream=stream)
        qkrope_run_3d_sharded(
            qkv, q_weight, k_weight, token_offset=token_offset, sumsq=sumsq_total,
            norm_elems_q=ne_q, norm_elems_k=ne_k, ppf=w.ppf, pph=w.pph, ppw=w.ppw,
            num_frame_channels=w.num_frame_channels, num_height_channels=w.num_height_channels,
            num_width_channels=w.num_width_channels, num_heads_q=Hq, num_heads_k=Hk,
            num_heads_v=Hv, head_dim=D, q_out=q_out, k_out=k_out, v_out=v_out, eps=w.eps,
            base=w.base, interleave=w.interleave, factor=w.factor, low=w.low, high=w.high,
            attention_factor=w.attention_factor, is_qk_norm=w.is_qk_norm,
            output_fp8=w.output_fp8, output_quant_scale=w.output_quant_scale,
            v_quant_scale=w.v_quant_scale, stream=stream)
        h, st = _handle_for(qkv.device), _stream(qkv.device, stream)
        L = lib()
        self._s = (L.qkrope_sumsq_3d, (h, _ptr(qkv), T, Hq, Hk, Hv, D, _ptr(sumsq), st))
        self._a = (L.qkrope_run_3d_sharded, (
            h, _ptr(qkv), _ptr(q_weight), _ptr(k_weight), T, int(token_offset), _ptr(sumsq_total),
            ne_q, ne_k, w.ppf, w.pph, w.ppw, w.num_frame_channels, w.num_height_channels,
            w.num_width_channels, Hq, Hk, Hv, D, float(w.eps), float(w.base), int(w.interleave),
            float(w.factor), float(w.low), float(w.high), float(w.attention_factor),
            int(w.is_qk_norm), int(w.output_fp8), float(w.output_quant_scale),
            float(w.v_quant_scale), _ptr(q_out), _ptr(k_out), _ptr(v_out), st))
        self._keep = (qkv, q_weight, k_weight, q_out, k_out, v_out, sumsq, sumsq_total)

    def sumsq(self) -> None:
        s = self._s[0](*self._s[1])
        if s != QKROPE_OK:
            _check(s, "qkrope_sumsq_3d")

    def apply(self) -> None:
        s = self._a[0](*self._a[1])
        if s != QKROPE_OK:
            _check(s, "qkrope_run_3d_sharded")

    def __call__(self) -> None:
        self.sumsq()
        self.apply()


_ACT_CODES = {torch.bfloat16: QKROPE_DTYPE_BF16, torch.float16: QKROPE_DTYPE_F16}


def _cam_rows(t: torch.Tensor, shape, name: str) -> int:
    """Token stride of a [B, N, H, D] view whose heads and dims are contiguous and whose batch
    stride is N token strides (the layout the C ABI takes)."""
    B, N, H, D = shape
    if t.dim() != 4 or tuple(t.shape) != (B, N, H, D):
        raise ValueError(f"{name} must be [batch, tokens, heads, head_dim] = {(B, N, H, D)}")
    if (H > 1 and t.stride(2) != D) or (D > 1 and t.stride(3) != 1):
        raise ValueError(f"{name} must have contiguous heads and dims")
    if N > 1:
        st = t.stride(1)
    else:                       # one token: its stride is the batch stride
        st = t.stride(0) if B > 1 else H * D
    if B > 1 and N > 0 and t.stride(0) != N * st:
        raise ValueError(f"{name}: batch stride must be tokens * token stride")
    return st


def _cam_out_rows(t: torch.Tensor, shape, name: str) -> int:
    """Row pitch of a [B, H, D, N] output view whose (b, h, d) rows are evenly spaced (contiguous,
    or the [..., :N] slice of padded rows): the out_row_stride the C ABI takes."""
    B, H, D, N = shape
    if t.dim() != 4 or tuple(t.shape) != (B, H, D, N):
        raise ValueError(f"{name} must be [batch, heads, head_dim, tokens] = {(B, H, D, N)}")
    if t.numel() == 0:
        return N                # nothing is written; torch's strides of an empty view vary
    rp = t.stride(2) if D > 1 else (t.stride(1) if H > 1 else (t.stride(0) if B > 1 else N))
    if ((N > 1 and t.stride(3) != 1) or rp < N or (H > 1 and t.stride(1) != D * rp) or
            (B > 1 and t.stride(0) != H * D * rp)):
        raise ValueError(f"{name} must have contiguous tokens and evenly spaced rows of at "
                         "least tokens elements (contiguous, or a slice of padded rows)")
    return rp


def qkrope_cam_prep(q, k, v, proj_q, proj_kv, rope_cos, rope_sin, k_scale, *, q_out, k_out,
                    v_out, inflation_sq=None, stream=None) -> None:
    """Camera prologue into caller-provided outputs: q, k, v [B, N, H, D] (bf16 or float16),
    proj_q / proj_kv float32 [B, N, 4, 4], rope_cos / rope_sin float32 [N, D/2]; q_out, k_out,
    v_out [B, H, D, N] of the activation dtype, contiguous or with one common row pitch (the
    [..., :N] slice of padded rows; a pitch that is a multiple of 64 starts every row on a
    128-byte line); inflation_sq contiguous float32 [B, H, N] or None."""
    if q.dim() != 4:
        raise ValueError("q must be [batch, tokens, heads, head_dim]")
    shape = tuple(q.shape)
    B, N, H, D = shape
    _c_ints(heads=H, head_dim=D)
    act = _ACT_CODES.get(q.dtype)
    if act is None or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a bfloat16 or float16 dtype")
    strides = [_cam_rows(t, shape, n) for t, n in ((q, "q"), (k, "k"), (v, "v"))]
    for t, n, want in ((proj_q, "proj_q", (B, N, 4, 4)), (proj_kv, "proj_kv", (B, N, 4, 4)),
                       (rope_cos, "rope_cos", (N, D // 2)), (rope_sin, "rope_sin", (N, D // 2))):
        if t.dtype != torch.float32 or tuple(t.shape) != want or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous float32 tensor of shape {want}")
    pitch = []
    for t, n in ((q_out, "q_out"), (k_out, "k_out"), (v_out, "v_out")):
        if t.dtype != q.dtype:
            raise ValueError(f"{n} must have the activation dtype")
        pitch.append(_cam_out_rows(t, (B, H, D, N), n))
    if len(set(pitch)) != 1:
        raise ValueError("q_out, k_out and v_out must share one row pitch")
    _same_device(q.device, k=k, v=v, proj_q=proj_q, proj_kv=proj_kv, rope_cos=rope_cos,
                 rope_sin=rope_sin, q_out=q_out, k_out=k_out, v_out=v_out,
                 inflation_sq=inflation_sq)
    if inflation_sq is not None and (inflation_sq.dtype != torch.float32 or
                                     tuple(inflation_sq.shape) != (B, H, N) or
                                     not inflation_sq.is_contiguous()):
        raise ValueError("inflation_sq must be a contiguous float32 [batch, heads, tokens] tensor")
    s = lib().qkrope_cam_prep(_handle_for(q.device), _ptr(q), _ptr(k), _ptr(v), act,
                              _ptr(proj_q), _ptr(proj_kv), _ptr(rope_cos), _ptr(rope_sin),
                              float(k_scale), B, N, H, D, strides[0], strides[1], strides[2],
                              _ptr(q_out), _ptr(k_out), _ptr(v_out), pitch[0], _ptr(inflation_sq),
                              _stream(q.device, stream))
    _check(s, "qkrope_cam_prep")


def cam_prep_func(q_normed, k_normed, v_raw, *, proj_q, proj_kv, rope_cos, rope_sin, k_scale):
    """vLLM-Omni's cam_prep_func signature: returns q_trans, k_trans, v_trans [B, H, D, N] and
    inflation_sq [B, H, N] (the library header states how the steps compose)."""
    B, N, H, D = q_normed.shape
    outs = [torch.empty((B, H, D, N), dtype=q_normed.dtype, device=q_normed.device)
            for _ in range(3)]
    infl = torch.empty((B, H, N), dtype=torch.float32, device=q_normed.device)
    qkrope_cam_prep(q_normed, k_normed, v_raw, proj_q, proj_kv, rope_cos, rope_sin, k_scale,
                    q_out=outs[0], k_out=outs[1], v_out=outs[2], inflation_sq=infl)
    return outs[0], outs[1], outs[2], infl


class PreparedCam:
    """One qkrope_cam_prep call marshalled once for repeated launches (tensors must stay alive
    and unmoved)."""

    def __init__(self, q, k, v, proj_q, proj_kv, rope_cos, rope_sin, k_scale, q_out, k_out,
                 v_out, inflation_sq, stream=None):
        qkrope_cam_prep(q, k, v, proj_q, proj_kv, rope_cos, rope_sin, k_scale, q_out=q_out,
                        k_out=k_out, v_out=v_out, inflation_sq=inflation_sq, stream=stream)
        B, N, H, D = q.shape
        st = [_cam_rows(t, tuple(q.shape), "x") for t in (q, k, v)]
        pitch = _cam_out_rows(q_out, (B, H, D, N), "q_out")
        self._fn = lib().qkrope_cam_prep
        self._args = (_handle_for(q.device), _ptr(q), _ptr(k), _ptr(v), _ACT_CODES[q.dtype],
                      _ptr(proj_q), _ptr(proj_kv), _ptr(rope_cos), _ptr(rope_sin),
                      float(k_scale), B, N, H, D, st[0], st[1], st[2], _ptr(q_out), _ptr(k_out),
                      _ptr(v_out), pitch, _ptr(inflation_sq), _stream(q.device, stream))
        self._keep = (q, k, v, proj_q, proj_kv, rope_cos, rope_sin, q_out, k_out, v_out,
                      inflation_sq)

    def __call__(self) -> None:
        s = self._fn(*self._args)
        if s != QKROPE_OK:
            _check(s, "qkrope_cam_prep")


def run_workload_3d(w, qkv, q_weight, k_weight, q_out=None, k_out=None, v_out=None):
    """fused_qk_rmsnorm_rope with the parameters of a 3D workload description."""
    return fused_qk_rmsnorm_rope(
        qkv, q_weight, k_weight, ppf=w.ppf, pph=w.pph, ppw=w.ppw,
        num_frame_channels=w.num_frame_channels, num_height_channels=w.num_height_channels,
        num_width_channels=w.num_width_channels, num_heads_q=w.num_heads_q,
        num_heads_k=w.num_heads_k, num_heads_v=w.num_heads_v, head_dim=w.head_dim, eps=w.eps,
        base=w.base, interleave=w.interleave, factor=w.factor, low=w.low, high=w.high,
        attention_factor=w.attention_factor, is_qk_norm=w.is_qk_norm, output_fp8=w.output_fp8,
        output_quant_scale=w.output_quant_scale, v_quant_scale=w.v_quant_scale,
        q_out=q_out, k_out=k_out, v_out=v_out)
