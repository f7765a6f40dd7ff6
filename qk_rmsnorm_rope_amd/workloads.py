"""Seeded synthetic workloads for the fused QK-RMSNorm + RoPE (+ V) prologue.

This module only draws inputs: shapes, seeds and value distributions. It holds none of the
prologue's arithmetic (no normalisation, no rotation, no quantisation), so the HIP path and the
fp64 oracle can both consume its arrays without sharing any method code.

Workload shapes follow the two API pages the prologue is built from:
  * vLLM-Omni "vllm_omni.diffusion.layers.fused_qk_norm_rope" (table form): q and k are
    [tokens, heads, head_dim], norm weights are [head_dim], the rope table is
    [tokens, rotary_dim] holding [cos(theta) | sin(theta)] in the activation dtype or float32.
  * FlashInfer "flashinfer.norm.fused_qk_rmsnorm_rope" (3D form): packed bf16 QKV
    [batch, seq_len, (Hq+Hk+Hv)*head_dim] with seq_len = ppf*pph*ppw, weights [H*head_dim].

Value recipe (stated once, used everywhere):
  * activations: numpy PCG64(seed).standard_normal in float32, times sigma, rounded to bf16 (RNE)
    or, for float16 table-form workloads, to IEEE binary16 (RNE);
  * norm weights: 1 + 0.1*N(0,1) drawn in float64, rounded to float32 then to the activation
    format (RNE);
  * rope table (table form only): theta_i = t * base**(-2i/rotary_dim) for token t, cos/sin taken
    in float64 and rounded to float32 (and then to bf16 or binary16 for a 16-bit table). The
    table is an input of the table form; the pages leave its contents to the caller.
  * camera prologue (vLLM-Omni "vllm_omni.diffusion.models.sana_wm.ucpe", cam_prep_func):
    q, k, v [B, N, H, D] drawn as activations (q and k stand for already-normalised values,
    unit RMS); proj_q and proj_kv are per-token rigid camera transforms [[R, t], [0, 0, 0, 1]]
    with R from a normalised N(0,1) quaternion and t = 0.5*N(0,1)^3, in float32; the split
    tables are cos/sin of theta_i = n * base**(-2i/D), float64 rounded to float32.
Every array is dense and contiguous, with no padding and no special values.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np
import torch

SEED_BASE = 20261203
_CHUNK = 1 << 24  # elements drawn per PCG64 call when filling large activations

# Role offsets added to a workload's seed, so each input has its own stream.
ROLE_QKV = 0   # packed qkv (3D form) or q (table form)
ROLE_K = 1     # k (table form)
ROLE_WQ = 2
ROLE_WK = 3
ROLE_V = 4     # v (camera prologue)
ROLE_PQ = 5    # proj_q
ROLE_PKV = 6   # proj_kv


@dataclass(frozen=True)
class TableWorkload:
    """Table-form problem: q, k [T, H, D] bf16 or float16; table [T, R] fp32 or 16-bit."""
    name: str
    num_tokens: int
    num_heads_q: int
    num_heads_k: int
    head_dim: int
    rotary_dim: int
    interleaved: bool
    table_dtype: str          # "f32", or the activation format "bf16" / "f16"
    seed: int
    eps: float = 1e-6
    base: float = 10000.0
    sigma: float = 1.0
    norm_mode: str = "per_head"   # "none" | "per_head" | "across_heads"
    act_dtype: str = "bf16"       # "bf16" | "f16": q, k and weights
    out_dtype: str = "act"        # "act" (the activation format) | "e4m3"
    out_scale: float = 1.0        # E4M3 outputs: codes of y * out_scale

    def with_(self, **kw) -> "TableWorkload":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class Rope3DWorkload:
    """3D-form problem: packed bf16 qkv [B, S, (Hq+Hk+Hv)*D], S = ppf*pph*ppw."""
    name: str
    batch: int
    ppf: int
    pph: int
    ppw: int
    num_frame_channels: int
    num_height_channels: int
    num_width_channels: int
    num_heads_q: int
    num_heads_k: int
    num_heads_v: int
    head_dim: int
    seed: int
    eps: float = 1e-6
    base: float = 10000.0
    interleave: bool = True
    factor: float = 1.0
    low: float = 0.0
    high: float = 0.0
    attention_factor: float = 1.0
    is_qk_norm: bool = True
    output_fp8: bool = False
    output_quant_scale: float = 1.0
    v_quant_scale: float = 1.0
    sigma: float = 1.0
    # > 1: the problem is one rank's share of a head-sharded run over this many ranks (the head
    # counts above are per rank); the across-heads norm spans head_shards times the rank's Q (K)
    # elements, taking the per-token sums of squares reduced over the ranks.
    head_shards: int = 1

    @property
    def seq_len(self) -> int:
        return self.ppf * self.pph * self.ppw

    @property
    def num_tokens(self) -> int:
        return self.batch * self.seq_len

    @property
    def row_elems(self) -> int:
        return (self.num_heads_q + self.num_heads_k + self.num_heads_v) * self.head_dim

    def with_(self, **kw) -> "Rope3DWorkload":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class CamWorkload:
    """Camera prologue: q, k, v [B, N, H, D]; projections [B, N, 4, 4]; tables [N, D/2] fp32.
    The N tokens form a ppf x pph x ppw latent grid; k_scale = D^-1/2 * (pph*ppw)^-1/2 (the page's
    D^-0.5 * spatial_tokens^-0.5 with the spatial tokens of one frame)."""
    name: str
    batch: int
    ppf: int
    pph: int
    ppw: int
    num_heads: int
    head_dim: int
    seed: int
    act_dtype: str = "bf16"
    base: float = 10000.0
    out_row_stride: int = 0     # elements between output rows (b, h, d); 0: num_tokens

    @property
    def num_tokens(self) -> int:
        return self.ppf * self.pph * self.ppw

    @property
    def out_pitch(self) -> int:
        return self.out_row_stride or self.num_tokens

    @property
    def k_scale(self) -> float:
        return float(self.head_dim ** -0.5 * (self.pph * self.ppw) ** -0.5)

    def with_(self, **kw) -> "CamWorkload":
        return dataclasses.replace(self, **kw)


# --- the five named workloads ------------------------------------------------------------------

# MiniMax-H3 geometry of the table form's half-split kernel (head_dim 128, rotary_dim 96).
TABLE_HALFSPLIT_T256 = TableWorkload(
    name="table_halfsplit_t256_h4_d128_r96_f32table", num_tokens=256, num_heads_q=4,
    num_heads_k=4, head_dim=128, rotary_dim=96, interleaved=False, table_dtype="f32",
    seed=SEED_BASE + 10)

# Boogu-Image style interleaved table form.
TABLE_INTERLEAVED_T4096 = TableWorkload(
    name="table_interleaved_t4096_h24_d128_bf16table", num_tokens=4096, num_heads_q=24,
    num_heads_k=24, head_dim=128, rotary_dim=128, interleaved=True, table_dtype="bf16",
    seed=SEED_BASE + 20)

# LTX-2 video self-attention shape: 15360 tokens, 32 heads of 128.
ROPE3D_ACROSS_S15360 = Rope3DWorkload(
    name="rope3d_across_interleaved_s15360_h32_d128", batch=1, ppf=16, pph=24, ppw=40,
    num_frame_channels=16, num_height_channels=56, num_width_channels=56,
    num_heads_q=32, num_heads_k=32, num_heads_v=32, head_dim=128, seed=SEED_BASE + 30)

# SANA-WM's 18480-token grid, NeoX pairing, FP8 E4M3 outputs.
ROPE3D_NEOX_FP8_S18480 = Rope3DWorkload(
    name="rope3d_neox_fp8_b2_s18480_h20_d64", batch=2, ppf=20, pph=33, ppw=28,
    num_frame_channels=16, num_height_channels=24, num_width_channels=24,
    num_heads_q=20, num_heads_k=20, num_heads_v=20, head_dim=64, seed=SEED_BASE + 40,
    interleave=False, output_fp8=True, output_quant_scale=0.5, v_quant_scale=0.25, sigma=2.0)

# Long-video YaRN, RoPE only.
ROPE3D_YARN_S122880 = Rope3DWorkload(
    name="rope3d_yarn_nonorm_s122880_h16_d256", batch=1, ppf=32, pph=48, ppw=80,
    num_frame_channels=64, num_height_channels=96, num_width_channels=96,
    num_heads_q=16, num_heads_k=16, num_heads_v=16, head_dim=256, seed=SEED_BASE + 50,
    factor=4.0, low=1.0, high=32.0, attention_factor=1.0 + 0.1 * float(np.log(4.0)),
    is_qk_norm=False)

# --- further measured workloads (beyond the five above) -----------------------------------------

# The interleaved table form at a token count whose working set (0.8 GB) exceeds the 256 MB
# memory-side cache, in bf16, in float16, and with E4M3 outputs.
TABLE_INTERLEAVED_T32768 = TABLE_INTERLEAVED_T4096.with_(
    name="table_interleaved_t32768_h24_d128_bf16table", num_tokens=32768, seed=SEED_BASE + 60)
TABLE_INTERLEAVED_T32768_F16 = TABLE_INTERLEAVED_T32768.with_(
    name="table_interleaved_t32768_h24_d128_f16", act_dtype="f16", table_dtype="f16",
    seed=SEED_BASE + 70)
TABLE_INTERLEAVED_T32768_E4M3 = TABLE_INTERLEAVED_T32768.with_(
    name="table_interleaved_t32768_h24_d128_e4m3out", out_dtype="e4m3", out_scale=0.5,
    table_dtype="f32", seed=SEED_BASE + 80)

# One rank of the 15360-token, 32-head problem sharded over 4 ranks by heads (8 Q, K and V
# heads per rank; across-heads norm over all 32).
ROPE3D_ACROSS_S15360_TP4 = ROPE3D_ACROSS_S15360.with_(
    name="rope3d_across_interleaved_s15360_h32_d128_tp4rank", num_heads_q=8, num_heads_k=8,
    num_heads_v=8, head_shards=4, seed=SEED_BASE + 90)

# The SANA-WM camera branch on the same 2 x 18480-token grid (two CFG branches), 20 heads of 64.
CAM_PREP_S18480 = CamWorkload(
    name="cam_prep_b2_s18480_h20_d64", batch=2, ppf=20, pph=33, ppw=28, num_heads=20,
    head_dim=64, seed=SEED_BASE + 100)

# The same camera prologue on a 16 x 32 x 36 grid (2 x 18432 tokens): N a multiple of 64, so
# every output row of [B, H, D, N] starts on a 128-byte line (at 18480 the row pitch, 36960
# bytes, is 96 mod 128 and the rows start at four phases). A comparison point for the layout's
# cost, not a target shape.
CAM_PREP_S18432 = CAM_PREP_S18480.with_(
    name="cam_prep_b2_s18432_h20_d64", ppf=16, pph=32, ppw=36, seed=SEED_BASE + 110)

# The 2 x 18480-token camera prologue writing into padded output rows of 18496 elements (a
# multiple of 64: every row starts on a 128-byte line), the layout a caller that can take a row
# pitch would choose; the same inputs and outputs as cam_prep_b2_s18480_h20_d64.
CAM_PREP_S18480_P18496 = CAM_PREP_S18480.with_(
    name="cam_prep_b2_s18480_h20_d64_pitch18496", out_row_stride=18496)

WORKLOADS = {w.name: w for w in (TABLE_HALFSPLIT_T256, TABLE_INTERLEAVED_T4096,
                                 ROPE3D_ACROSS_S15360, ROPE3D_NEOX_FP8_S18480,
                                 ROPE3D_YARN_S122880, TABLE_INTERLEAVED_T32768,
                                 TABLE_INTERLEAVED_T32768_F16, TABLE_INTERLEAVED_T32768_E4M3,
                                 ROPE3D_ACROSS_S15360_TP4, CAM_PREP_S18480,
                                 CAM_PREP_S18432, CAM_PREP_S18480_P18496)}


# --- drawing -----------------------------------------------------------------------------------

def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


_TORCH_DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def bf16_normal(seed: int, n: int, sigma: float = 1.0, dtype: str = "bf16") -> torch.Tensor:
    """n draws of sigma*N(0,1) as a flat CPU tensor (float32 draws, RNE to bf16, or to float16
    with dtype="f16")."""
    rng = _rng(seed)
    out = torch.empty(n, dtype=_TORCH_DTYPES[dtype])
    for start in range(0, n, _CHUNK):
        m = min(_CHUNK, n - start)
        chunk = rng.standard_normal(m, dtype=np.float32)
        if sigma != 1.0:
            chunk *= np.float32(sigma)
        out[start:start + m] = torch.from_numpy(chunk).to(out.dtype)
    return out


def bf16_weights(seed: int, n: int, dtype: str = "bf16") -> torch.Tensor:
    """Norm weights 1 + 0.1*N(0,1), drawn in float64, as a CPU bfloat16 (or float16) tensor."""
    w = 1.0 + 0.1 * _rng(seed).standard_normal(n)
    return torch.from_numpy(w.astype(np.float32)).to(_TORCH_DTYPES[dtype])


def rope_table(num_tokens: int, rotary_dim: int, base: float, dtype: str) -> torch.Tensor:
    """[T, R] table: row t = [cos(theta_0..theta_{R/2-1}) | sin(...)], theta_i = t*base^(-2i/R)."""
    half = rotary_dim // 2
    inv = base ** (-(2.0 * np.arange(half, dtype=np.float64)) / rotary_dim)
    theta = np.arange(num_tokens, dtype=np.float64)[:, None] * inv[None, :]
    tab = np.concatenate([np.cos(theta), np.sin(theta)], axis=1).astype(np.float32)
    t = torch.from_numpy(np.ascontiguousarray(tab))
    if dtype not in _TORCH_DTYPES:
        raise ValueError(f"table dtype {dtype!r}")
    return t.to(_TORCH_DTYPES[dtype])


def table_inputs(w: TableWorkload) -> dict:
    """CPU tensors for a table-form workload: q, k [T,H,D] (bf16 or float16); weights; table."""
    T, D, a = w.num_tokens, w.head_dim, w.act_dtype
    q = bf16_normal(w.seed + ROLE_QKV, T * w.num_heads_q * D, w.sigma, a).view(T, w.num_heads_q, D)
    k = bf16_normal(w.seed + ROLE_K, T * w.num_heads_k * D, w.sigma, a).view(T, w.num_heads_k, D)
    wlen_q = D if w.norm_mode != "across_heads" else w.num_heads_q * D
    wlen_k = D if w.norm_mode != "across_heads" else w.num_heads_k * D
    return dict(q=q, k=k,
                q_weight=bf16_weights(w.seed + ROLE_WQ, wlen_q, a),
                k_weight=bf16_weights(w.seed + ROLE_WK, wlen_k, a),
                rope_table=rope_table(T, w.rotary_dim, w.base, w.table_dtype))


def rope3d_inputs(w: Rope3DWorkload) -> dict:
    """CPU tensors for a 3D workload: qkv [B, S, (Hq+Hk+Hv)*D] bf16 and the two weights."""
    qkv = bf16_normal(w.seed + ROLE_QKV, w.num_tokens * w.row_elems, w.sigma)
    return dict(qkv=qkv.view(w.batch, w.seq_len, w.row_elems),
                q_weight=bf16_weights(w.seed + ROLE_WQ, w.num_heads_q * w.head_dim),
                k_weight=bf16_weights(w.seed + ROLE_WK, w.num_heads_k * w.head_dim))


def rigid_transforms(seed: int, count: int) -> torch.Tensor:
    """count float32 4x4 matrices [[R, t], [0, 0, 0, 1]]: R from a normalised N(0,1)
    quaternion, t = 0.5*N(0,1)^3 (drawn in float64)."""
    rng = _rng(seed)
    qt = rng.standard_normal((count, 4))
    qt /= np.linalg.norm(qt, axis=1, keepdims=True)
    w, x, y, z = qt.T
    M = np.zeros((count, 4, 4))
    M[:, 0, 0] = 1 - 2 * (y * y + z * z)
    M[:, 0, 1] = 2 * (x * y - w * z)
    M[:, 0, 2] = 2 * (x * z + w * y)
    M[:, 1, 0] = 2 * (x * y + w * z)
    M[:, 1, 1] = 1 - 2 * (x * x + z * z)
    M[:, 1, 2] = 2 * (y * z - w * x)
    M[:, 2, 0] = 2 * (x * z - w * y)
    M[:, 2, 1] = 2 * (y * z + w * x)
    M[:, 2, 2] = 1 - 2 * (x * x + y * y)
    M[:, :3, 3] = 0.5 * rng.standard_normal((count, 3))
    M[:, 3, 3] = 1.0
    return torch.from_numpy(M.astype(np.float32))


def cam_inputs(w: CamWorkload) -> dict:
    """CPU tensors for a camera-prologue workload: q, k, v [B, N, H, D]; proj_q, proj_kv
    [B, N, 4, 4] float32; rope_cos, rope_sin [N, D/2] float32."""
    B, N, H, D, a = w.batch, w.num_tokens, w.num_heads, w.head_dim, w.act_dtype
    shape = (B, N, H, D)
    n = B * N * H * D
    tab = rope_table(N, D, w.base, "f32")
    return dict(q=bf16_normal(w.seed + ROLE_QKV, n, 1.0, a).view(shape),
                k=bf16_normal(w.seed + ROLE_K, n, 1.0, a).view(shape),
                v=bf16_normal(w.seed + ROLE_V, n, 1.0, a).view(shape),
                proj_q=rigid_transforms(w.seed + ROLE_PQ, B * N).view(B, N, 4, 4),
                proj_kv=rigid_transforms(w.seed + ROLE_PKV, B * N).view(B, N, 4, 4),
                rope_cos=tab[:, :D // 2].contiguous(), rope_sin=tab[:, D // 2:].contiguous())
