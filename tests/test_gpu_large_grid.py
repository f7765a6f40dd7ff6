"""Calls whose grid exceeds what one dispatch may hold (2^32 - 1 lanes), against the fp64 oracle.

The library runs such a call as several launches over consecutive token ranges. With 64-lane
workgroups (one head of head_dim 8 per region in the table form, one of 64 in the 3D form) a
launch covers at most 2^26 - 1 tokens, so a call past 2^26 tokens takes two. The inputs repeat a
seeded block of tokens along the token axis (every output token depends only on its own row and,
in the 3D form, its position), and the outputs are compared with the oracle on sampled tokens:
both ends, the seam between the two launches, and random ones.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from parity import check_3d_outputs, check_table_outputs

pytestmark = pytest.mark.gpu

qr = pytest.importorskip("qk_rmsnorm_rope_amd")
from qk_rmsnorm_rope_amd import workloads as wl  # noqa: E402

DEV = "cuda"
SEAM = ((1 << 32) - 1) // 64        # first token of the second launch (64-lane workgroups)
BLOCK = 4096                        # tokens in the seeded block that the inputs repeat


def sampled(T, seed):
    rng = np.random.default_rng(seed)
    picks = {0, 1, BLOCK - 1, BLOCK, SEAM - 2, SEAM - 1, SEAM, SEAM + 1, T - 2, T - 1}
    picks |= set(rng.integers(0, T, 40).tolist())
    return np.array(sorted(p for p in picks if 0 <= p < T))


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("interleaved", [True, False])
def test_table_form_past_one_grid(interleaved):
    T = (1 << 26) + 3001
    small = wl.TableWorkload(name="table_two_launches", num_tokens=BLOCK, num_heads_q=1,
                             num_heads_k=1, head_dim=8, rotary_dim=8, interleaved=interleaved,
                             table_dtype="f32", seed=wl.SEED_BASE + 300, norm_mode="per_head")
    inp = wl.table_inputs(small)
    reps = -(-T // BLOCK)
    q = inp["q"].to(DEV).repeat(reps, 1, 1)[:T]
    k = inp["k"].to(DEV).repeat(reps, 1, 1)[:T]
    tab = inp["rope_table"].to(DEV).repeat(reps, 1)[:T]
    wq, wk = inp["q_weight"].to(DEV), inp["k_weight"].to(DEV)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    print(f"\ntable form, {T} tokens, interleaved={interleaved}", flush=True)
    qr.qkrope_run_table(q, k, wq, wk, tab, small.eps, q_out=qo, k_out=ko, rotary_dim=8,
                        interleaved=interleaved, norm_mode="per_head")
    torch.cuda.synchronize()
    tokens = sampled(T, 1)
    rows = tokens % BLOCK
    rq, rk = oracle.run_table(inp["q"][rows], inp["k"][rows], inp["q_weight"], inp["k_weight"],
                              inp["rope_table"][rows], small.eps, rotary_dim=8,
                              interleaved=interleaved, norm_mode="per_head")
    idx = torch.as_tensor(tokens, device=DEV)
    check_table_outputs(small.name, qo[idx], ko[idx], rq, rk)


def test_3d_form_past_one_grid():
    # one sequence of 16x16x16 positions is the repeated block; 16385 sequences
    small = wl.Rope3DWorkload(name="rope3d_two_launches", batch=1, ppf=16, pph=16, ppw=16,
                              num_frame_channels=16, num_height_channels=24,
                              num_width_channels=24, num_heads_q=1, num_heads_k=1,
                              num_heads_v=1, head_dim=64, seed=wl.SEED_BASE + 301,
                              interleave=False)
    big = small.with_(batch=16385)
    T = big.num_tokens
    assert T > SEAM
    inp = wl.rope3d_inputs(small)
    block = inp["qkv"].reshape(BLOCK, small.row_elems)
    qkv = block.to(DEV).repeat(big.batch, 1).view(big.batch, BLOCK, small.row_elems)
    wq, wk = inp["q_weight"].to(DEV), inp["k_weight"].to(DEV)
    print(f"\n3D form, {T} tokens", flush=True)
    outs = qr.run_workload_3d(big, qkv, wq, wk)
    sums = qr.qkrope_sumsq_3d(qkv.view(T, -1), num_heads_q=1, num_heads_k=1, num_heads_v=1,
                              head_dim=64)
    torch.cuda.synchronize()
    tokens = sampled(T, 2)
    parts = [oracle.run_3d_workload(big, block[t % BLOCK:t % BLOCK + 1], inp["q_weight"],
                                    inp["k_weight"], token_offset=int(t)) for t in tokens]
    ref = tuple(np.concatenate([p[i] for p in parts]) for i in range(3))
    check_3d_outputs(big, outs, ref, tokens=tokens)
    ref_sums = oracle.sumsq_3d(block[tokens % BLOCK], num_heads_q=1, num_heads_k=1,
                               num_heads_v=1, head_dim=64)
    got = sums[torch.as_tensor(tokens, device=DEV)].cpu().numpy()
    np.testing.assert_allclose(got, ref_sums, rtol=1e-5)
    del outs
    torch.cuda.empty_cache()
    # the head-sharded apply over the same tokens, from global token 5 on, with the sums above:
    # each launch reads its own range of the sums and continues the positions
    off = 5
    so = [torch.empty((T, 1, 64), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    print("sharded apply", flush=True)
    qr.qkrope_run_3d_sharded(qkv.view(T, -1), wq, wk, token_offset=off, sumsq=sums,
                             norm_elems_q=64, norm_elems_k=64, ppf=big.ppf, pph=big.pph,
                             ppw=big.ppw, num_frame_channels=big.num_frame_channels,
                             num_height_channels=big.num_height_channels,
                             num_width_channels=big.num_width_channels, num_heads_q=1,
                             num_heads_k=1, num_heads_v=1, head_dim=64, eps=big.eps,
                             base=big.base, interleave=big.interleave, q_out=so[0], k_out=so[1],
                             v_out=so[2])
    torch.cuda.synchronize()
    parts = [oracle.run_3d_workload(big, block[t % BLOCK:t % BLOCK + 1], inp["q_weight"],
                                    inp["k_weight"], token_offset=int(t) + off) for t in tokens]
    ref = tuple(np.concatenate([p[i] for p in parts]) for i in range(3))
    check_3d_outputs(big, so, ref, tokens=tokens)
