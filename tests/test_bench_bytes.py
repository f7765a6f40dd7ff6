"""The algorithmic bytes bench.py divides by a kernel's time to get its GB/s, per named workload.

Each figure is the bytes the method must move once: activations and tables read, outputs
written, norm weights read once. The expected values are written out from the workloads'
shapes here (the same numbers the design notes tabulate), so a change to the byte model or to
a workload's shape shows up as a failure.
"""
from __future__ import annotations

import pytest

import bench
from qk_rmsnorm_rope_amd import workloads as wl

EXPECTED = {
    # table: q, k [T, H, D] bf16 read and written, the table [T, R] once, two [D] weights
    "table_halfsplit_t256_h4_d128_r96_f32table": 256 * 8 * 128 * 2 * 2 + 256 * 96 * 4 + 2 * 128 * 2,
    "table_interleaved_t4096_h24_d128_bf16table":
        4096 * 48 * 128 * 2 * 2 + 4096 * 128 * 2 + 2 * 128 * 2,
    "table_interleaved_t32768_h24_d128_bf16table":
        32768 * 48 * 128 * 2 * 2 + 32768 * 128 * 2 + 2 * 128 * 2,
    "table_interleaved_t32768_h24_d128_f16": 32768 * 48 * 128 * 2 * 2 + 32768 * 128 * 2 + 2 * 128 * 2,
    # E4M3 outputs: one byte per output element; the fp32 table
    "table_interleaved_t32768_h24_d128_e4m3out":
        32768 * 48 * 128 * (2 + 1) + 32768 * 128 * 4 + 2 * 128 * 2,
    # 3D: packed qkv read, q, k, v written, [H*D] weights for Q and K once
    "rope3d_across_interleaved_s15360_h32_d128": 15360 * 96 * 128 * 2 * 2 + 64 * 128 * 2,
    "rope3d_neox_fp8_b2_s18480_h20_d64": 36960 * 60 * 64 * (2 + 1) + 40 * 64 * 2,
    "rope3d_yarn_nonorm_s122880_h16_d256": 122880 * 48 * 256 * 2 * 2,
    # one rank of four head shards: its 8+8+8 heads, its weights, the [T, 2] fp32 sums
    "rope3d_across_interleaved_s15360_h32_d128_tp4rank":
        15360 * 24 * 128 * 2 * 2 + 16 * 128 * 2 + 15360 * 8,
    # camera: q, k, v in and out, two 4x4 fp32 matrices per (b, n), [N, D/2] cos and sin once,
    # inflation_sq [B, H, N] fp32 out
    "cam_prep_b2_s18480_h20_d64":
        36960 * (12 * 20 * 64 + 2 * 64) + 18480 * 2 * 32 * 4 + 36960 * 20 * 4,
    "cam_prep_b2_s18432_h20_d64":
        36864 * (12 * 20 * 64 + 2 * 64) + 18432 * 2 * 32 * 4 + 36864 * 20 * 4,
    # padded output rows: the padding is neither read nor written
    "cam_prep_b2_s18480_h20_d64_pitch18496":
        36960 * (12 * 20 * 64 + 2 * 64) + 18480 * 2 * 32 * 4 + 36960 * 20 * 4,
}


def test_every_named_workload_is_covered():
    assert set(EXPECTED) == set(wl.WORKLOADS)


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_algorithmic_bytes(name):
    assert bench.algorithmic_bytes(wl.WORKLOADS[name]) == EXPECTED[name]


def test_sums_kernel_bytes_of_the_sharded_rank():
    w = wl.WORKLOADS["rope3d_across_interleaved_s15360_h32_d128_tp4rank"]
    assert bench.sumsq_bytes(w) == 15360 * (16 * 128 * 2 + 8) == 63_037_440


def test_across_heads_table_weights_are_counted_per_head():
    w = wl.WORKLOADS["table_interleaved_t4096_h24_d128_bf16table"].with_(norm_mode="across_heads")
    per_head = bench.algorithmic_bytes(w.with_(norm_mode="per_head"))
    assert bench.algorithmic_bytes(w) - per_head == (48 - 2) * 128 * 2
    assert per_head - bench.algorithmic_bytes(w.with_(norm_mode="none")) == 2 * 128 * 2
