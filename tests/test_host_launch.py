"""The host side of the C ABI (qkrope_api.cpp) on the CPU: launch shapes and launch loops.

A small C++ program compiles the library's own host source with the kernel launchers and the
few HIP runtime calls it makes replaced by stubs that record each launch (its kernel key,
launch shape, token range and input offset) instead of running it. The entry points then run
unchanged on fake, never-dereferenced device addresses. This pins:
  * the launch shape each named workload gets (the shapes the kernels were tuned for);
  * the region split (three workgroups per token) where it applies, and only there;
  * calls whose grid exceeds one dispatch: how many launches, their token ranges, grid sizes,
    pointer offsets and position offsets, at sizes no GPU test allocates.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "qk_rmsnorm_rope_amd", "csrc")

DRIVER = r"""
#include "qkrope_api.cpp"
#include "qkrope_api_cam.cpp"

#include <cstdio>
#include <cstdlib>
#include <cstring>

// ---- stubs: HIP runtime queries (no device here) and kernel launchers that record ----------
hipError_t hipGetDevice(int *d) { *d = 0; return hipSuccess; }
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipGetDeviceCount(int *n) { *n = 0; return hipSuccess; }
hipError_t hipGetDeviceProperties(hipDeviceProp_t *, int) { return hipErrorNoDevice; }
const char *hipGetErrorString(hipError_t) { return "stub"; }

static uintptr_t g_base;     // the call's first input, to print offsets from

static hipError_t rec(const char *kind, const qkrope::KernelKey &k, const qkrope::LaunchShape &s,
                      const qkrope::KernelArgs &a)
{
    std::printf("launch %s threads=%d slots=%d su=%d tpw=%d split=%d blocks=%lld tpl=%d "
                "pairing=%d norm=%d fp8=%d ntok=%lld toff=%u in0=%llu xcd=%u\n",
                kind, s.threads, s.slots, (int)s.slot_uniform, s.tpw, (int)s.split,
                (long long)s.blocks, k.head_dim_tpl, k.pairing, k.norm, (int)k.fp8,
                (long long)a.num_tokens, a.token_offset,
                (unsigned long long)(reinterpret_cast<uintptr_t>(a.in[0]) - g_base), a.xcd_group);
    return hipSuccess;
}
#define STUB(name) \
    hipError_t qkrope::name(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t) \
    { return rec(#name, k, s, a); }
STUB(launch_3d_d64) STUB(launch_3d_d128) STUB(launch_3d_d256)
STUB(launch_table_interleaved_bf16) STUB(launch_table_halfsplit_bf16)
STUB(launch_table_interleaved_f16) STUB(launch_table_halfsplit_f16)
STUB(launch_table_halfsplit_any_bf16) STUB(launch_table_halfsplit_any_f16)
hipError_t qkrope::launch_sumsq(const SumsqArgs &, int64_t tokens, int threads, hipStream_t)
{
    std::printf("launch sumsq threads=%d tokens=%lld\n", threads, (long long)tokens);
    return hipSuccess;
}

hipError_t qkrope::launch_cam(const CamArgs &a, int act, int cpl, int64_t blocks, int lds_bytes,
                              hipStream_t)
{
    std::printf("launch cam act=%d cpl=%d lanes=%d hpg=%d groups=%d tiles=%d tiles_padded=%d "
                "xcd=%u blocks=%lld lds=%d row_chunks=%d vec=%d\n",
                act, cpl, a.lanes_per_token, a.heads_per_group, a.groups, a.tiles, a.tiles_padded,
                a.xcd_group, (long long)blocks, lds_bytes, a.row_chunks, a.vec_store);
    return hipSuccess;
}

static void *at(int k) { return reinterpret_cast<void *>((uintptr_t(1) << 40) + (uintptr_t(k) << 38)); }

int main(int argc, char **argv)
{
    qkrope_ctx ctx{0, 256, "gfx950"};
    qkrope_handle h = &ctx;
    const char *form = argv[1];
    double v[40] = {0};
    for (int i = 2; i < argc && i < 42; ++i) v[i - 2] = std::atof(argv[i]);
    auto I = [&](int i) { return (long long)v[i]; };
    g_base = reinterpret_cast<uintptr_t>(at(0));
    int st;
    if (!std::strcmp(form, "3d")) {
        // T ppf pph ppw cf ch cw Hq Hk Hv D interleave is_qk_norm fp8 token_offset use_sumsq
        // eps base factor low high attention_factor out_scale v_scale qkv_shift_bytes
        // q_out_mode (0: own buffer, 1: inside qkv)
        const long long T = I(0);
        const int D = (int)I(10);
        const bool sums = I(15) != 0;
        const void *qkv = static_cast<const char *>(at(0)) + I(24);
        void *qo = I(25) == 1 ? static_cast<char *>(at(0)) + 4096 : at(1);
        st = qkrope_run_3d_sharded(h, qkv, at(4), at(5), T, I(14), sums ? (const float *)at(6) : nullptr,
                                   I(7) * D, I(8) * D, (int)I(1), (int)I(2), (int)I(3), (int)I(4),
                                   (int)I(5), (int)I(6), (int)I(7), (int)I(8), (int)I(9), D, v[16],
                                   v[17], (int)I(11), v[18], v[19], v[20], v[21], (int)I(12),
                                   (int)I(13), v[22], v[23], qo, at(2), at(3), nullptr);
    } else if (!std::strcmp(form, "cam")) {
        // B N H D act
        const long long B = I(0), N = I(1);
        const int H = (int)I(2), D = (int)I(3);
        const long long s = (long long)H * D;
        st = qkrope_cam_prep(h, at(0), at(1), at(2), (int)I(4), (const float *)at(3),
                             (const float *)at(4), (const float *)at(5), (const float *)at(6),
                             0.5f, B, N, H, D, s, s, s, at(7), at(8), at(9), (float *)at(10),
                             nullptr);
    } else {
        // T Hq Hk D R interleaved norm_mode act out tdt q_stride eps out_scale q_shift_bytes
        // q_out_mode (0: own buffer, 1: q itself, 2: q shifted by 16 bytes)
        const long long T = I(0);
        const int Hq = (int)I(1), Hk = (int)I(2), D = (int)I(3), R = (int)I(4);
        const long long qs = I(10) ? I(10) : (long long)Hq * D;
        const void *q = static_cast<const char *>(at(0)) + I(13);
        void *qo = I(14) == 1 ? const_cast<void *>(q)
                 : I(14) == 2 ? static_cast<char *>(const_cast<void *>(q)) + 16 : at(4);
        st = qkrope_run_table_ex(h, q, at(1), at(6), at(7), at(2), at(3), (int)I(9), (int)I(7),
                                 (int)I(8), v[12], v[11], T, Hq, Hk, D, R, (int)I(5), (int)I(6), qs,
                                 (long long)Hk * D, R / 2, R / 2, qo, at(5), qs,
                                 (long long)Hk * D, nullptr);
    }
    std::printf("status %d %s\n", st, qkrope_last_error());
    return 0;
}
"""


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    d = tmp_path_factory.mktemp("launch")
    src, exe = d / "launch_check.cpp", d / "launch_check"
    src.write_text(DRIVER)
    subprocess.run(["g++", "-std=c++17", "-O1", "-w", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True, capture_output=True, text=True)
    return str(exe)


def run(driver, *args):
    """The recorded launches (dicts of their fields) and the call's status."""
    out = subprocess.run([driver, *map(str, args)], capture_output=True, text=True, timeout=60,
                         check=True).stdout.splitlines()
    launches = []
    for line in out:
        if line.startswith("launch "):
            parts = line.split()
            rec = {"kind": parts[1]}
            rec.update({k: v for k, v in (p.split("=") for p in parts[2:])})
            launches.append({k: (v if k == "kind" else int(v)) for k, v in rec.items()})
    status = int(out[-1].split()[1])
    return launches, status


def run_3d(driver, T, grid, ch, heads, D, interleave=1, norm=1, fp8=0, offset=0, sums=0,
           eps=1e-6, base=1e4, factor=1.0, low=0.0, high=0.0, af=1.0, oqs=1.0, vqs=1.0,
           shift=0, q_out_mode=0):
    return run(driver, "3d", T, *grid, *ch, *heads, D, interleave, norm, fp8, offset, sums, eps,
               base, factor, low, high, af, oqs, vqs, shift, q_out_mode)


def run_table(driver, T, Hq, Hk, D, R, inter=1, norm=1, act=0, out=0, tdt=1, q_stride=0,
              eps=1e-6, out_scale=1.0, shift=0, q_out_mode=0):
    return run(driver, "table", T, Hq, Hk, D, R, inter, norm, act, out, tdt, q_stride, eps,
               out_scale, shift, q_out_mode)


def test_named_3d_workloads_get_their_tuned_shapes(driver):
    # 15360 x 3x32 x 128, across heads: one token per 512-lane workgroup, one chunk per region
    (l,), st = run_3d(driver, 15360, (16, 24, 40), (16, 56, 56), (32, 32, 32), 128)
    assert st == 0 and l["kind"] == "launch_3d_d128"
    assert (l["threads"], l["slots"], l["su"], l["tpw"], l["split"]) == (512, 1, 1, 1, 0)
    assert l["blocks"] == 15360 and l["xcd"] == 16
    # 2 x 18480 x 3x20 x 64, NeoX, FP8: two tokens of 160 lanes per 320-lane workgroup
    (l,), st = run_3d(driver, 36960, (20, 33, 28), (16, 24, 24), (20, 20, 20), 64, interleave=0,
                      fp8=1)
    assert st == 0 and (l["threads"], l["tpw"], l["split"], l["fp8"]) == (320, 2, 0, 1)
    assert l["blocks"] == 36960 // 2
    # 122880 x 3x16 x 256, no norm: one region of one token per workgroup (three per token)
    (l,), st = run_3d(driver, 122880, (32, 48, 80), (64, 96, 96), (16, 16, 16), 256, norm=0)
    assert st == 0 and (l["threads"], l["split"], l["norm"]) == (512, 1, 0)
    assert l["blocks"] == 3 * 122880


@pytest.mark.parametrize("norm,fp8,heads", [(1, 0, (16, 16, 16)), (0, 1, (16, 16, 16)),
                                            (0, 0, (4, 4, 4))])
def test_region_split_only_without_norm_for_16_bit_outputs_and_wide_rows(driver, norm, fp8,
                                                                         heads):
    (l,), st = run_3d(driver, 1536, (4, 4, 96), (64, 96, 96), heads, 256, norm=norm, fp8=fp8)
    assert st == 0 and l["split"] == 0 and l["blocks"] == 1536 // l["tpw"]


def test_named_table_workloads_get_their_tuned_shapes(driver):
    # 4096 x 2x24 x 128, interleaved, bf16 table: 384 lanes (16 per head), one token each
    (l,), st = run_table(driver, 4096, 24, 24, 128, 128, tdt=0)
    assert st == 0 and l["kind"] == "launch_table_interleaved_bf16"
    assert (l["threads"], l["slots"], l["tpw"], l["split"], l["tpl"]) == (384, 1, 1, 0, 0)
    # E4M3 outputs at head_dim == rotary_dim == 128 take the compile-time head geometry
    (l,), st = run_table(driver, 32768, 24, 24, 128, 128, out=3)
    assert st == 0 and l["tpl"] == 128 and l["fp8"] == 1
    # half-split with rotary_dim % 16 != 0 exchanges partners through LDS
    (l,), st = run_table(driver, 64, 2, 2, 128, 72, inter=0)
    assert st == 0 and l["kind"] == "launch_table_halfsplit_any_bf16"


def test_region_split_past_one_grid_runs_as_two_launches(driver):
    # 512-lane workgroups, three per token: one launch takes floor((2^32 - 1) / 512 / 3) tokens
    per = ((1 << 32) - 1) // 512 // 3
    T = per + 3001
    heads, D = (32, 32, 16), 128
    row = sum(heads) * D
    ls, st = run_3d(driver, T, (1, 1, 7), (32, 48, 48), heads, D, norm=0, offset=11)
    assert st == 0 and len(ls) == 2
    a, b = ls
    assert a["split"] == b["split"] == 1
    assert (a["ntok"], b["ntok"]) == (per, 3001)
    assert (a["blocks"], b["blocks"]) == (3 * per, 3 * 3001)
    assert (a["toff"], b["toff"]) == (11, 11 + per)
    assert (a["in0"], b["in0"]) == (0, per * row * 2)
    assert a["blocks"] * a["threads"] <= (1 << 32) - 1


@pytest.mark.parametrize("with_table", [False, True])
def test_one_token_per_workgroup_past_one_grid(driver, with_table):
    # 64-lane workgroups (one head of 64 per region), with the across-heads sums passed in
    heads = (1, 1, 1)
    per = ((1 << 32) - 1) // 64
    T = 2 * per + 5
    ls, st = run_3d(driver, T, (1, 1, 5), (16, 24, 24), heads, 64, offset=3, sums=1)
    assert st == 0 and [l["ntok"] for l in ls] == [per, per, 5]
    assert [l["toff"] for l in ls] == [3, 3 + per, 3 + 2 * per]
    assert [l["in0"] for l in ls] == [0, per * 3 * 64 * 2, 2 * per * 3 * 64 * 2]
    assert all(l["blocks"] * l["threads"] <= (1 << 32) - 1 for l in ls)
    if with_table:   # the table form's rows, past one grid at 64-lane workgroups
        T2 = per + 9
        ls, st = run_table(driver, T2, 1, 1, 8, 8)
        assert st == 0 and [l["ntok"] for l in ls] == [per, 9]
        assert [l["in0"] for l in ls] == [0, per * 8 * 2]


def test_shapes_past_the_largest_rows_are_refused_before_any_launch(driver):
    ls, st = run_3d(driver, 8, (1, 2, 4), (32, 48, 48), (129, 128, 128), 128)
    assert ls == [] and st == 2
    ls, st = run_table(driver, 4, 257, 1, 128, 128)
    assert ls == [] and st == 2


def test_camera_prologue_launch(driver):
    # 2 x 18480 x 20 heads x 64: groups of 2 heads, 64-token tiles padded to a multiple of 8 so
    # each XCD takes a contiguous eighth, 16-byte stores (N % 8 == 0)
    (l,), st = run(driver, "cam", 2, 18480, 20, 64, 0)
    assert st == 0
    assert (l["cpl"], l["lanes"], l["hpg"], l["groups"]) == (1, 8, 2, 10)
    assert (l["tiles"], l["tiles_padded"], l["xcd"]) == (289, 296, 37)
    assert (l["blocks"], l["lds"], l["row_chunks"], l["vec"]) == (2 * 296 * 10, 16384, 8, 1)
    # head_dim 128: two chunks per lane, one head per group; odd heads split as evenly as can be
    (l,), st = run(driver, "cam", 1, 1000, 3, 128, 2)
    assert st == 0 and (l["cpl"], l["hpg"], l["groups"], l["row_chunks"]) == (2, 1, 3, 16)
    (l,), st = run(driver, "cam", 1, 1000, 3, 64, 0)
    assert st == 0 and (l["hpg"], l["groups"]) == (2, 2)
    # head_dim 40: five chunks in a power-of-two LDS row; N % 8 != 0 stores elements
    (l,), st = run(driver, "cam", 1, 301, 2, 40, 0)
    assert st == 0 and (l["lanes"], l["row_chunks"], l["vec"]) == (8, 8, 0)
    # fewer than 8 tiles: plain block order
    (l,), st = run(driver, "cam", 3, 200, 4, 64, 0)
    assert st == 0 and (l["tiles"], l["tiles_padded"], l["xcd"]) == (4, 4, 0)


def test_camera_prologue_grid_limit(driver):
    # one head of 64 (512-lane workgroups): 2^23 tiles fill 2^32 lanes; tiles are padded to a
    # multiple of 8, so one tile fewer is still refused and eight fewer fit
    for n in ((1 << 29), (1 << 29) - 64):
        ls, st = run(driver, "cam", 1, n, 1, 64, 0)
        assert ls == [] and st == 2
    (l,), st = run(driver, "cam", 1, (1 << 29) - 8 * 64, 1, 64, 0)
    assert st == 0 and l["blocks"] * 64 * l["lanes"] < (1 << 32)


# --- argument validation: each contract rule, on the CPU (status 1 invalid, 2 unsupported) ------

G3 = dict(T=120, grid=(2, 3, 4), ch=(32, 48, 48), heads=(4, 2, 2), D=128)


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(eps=-1.0), 1), (dict(eps=float("nan")), 1), (dict(base=0.0), 1),
    (dict(base=float("inf")), 1), (dict(factor=0.0), 1), (dict(factor=2.0, low=3.0, high=3.0), 1),
    (dict(factor=2.0, low=0.0, high=float("inf")), 1), (dict(af=1.1), 1),
    (dict(factor=2.0, high=8.0, af=float("nan")), 1), (dict(factor=2.0, high=8.0, af=1.1), 0),
    (dict(fp8=1, oqs=0.0), 1), (dict(fp8=1, vqs=-1.0), 1), (dict(fp8=1, oqs=0.5, vqs=2.0), 0),
    (dict(D=96, ch=(32, 32, 32)), 1), (dict(ch=(31, 49, 48)), 1), (dict(ch=(32, 48, 40)), 1),
    (dict(grid=(0, 3, 4)), 1), (dict(offset=-1), 1), (dict(offset=(1 << 31) - 100), 2),
    (dict(shift=8), 2), (dict(q_out_mode=1), 1),
], ids=lambda v: str(v))
def test_3d_argument_rules(driver, kw, status):
    args = {**G3, **kw}
    ls, st = run_3d(driver, args.pop("T"), args.pop("grid"), args.pop("ch"), args.pop("heads"),
                    args.pop("D"), **args)
    assert st == status
    assert (ls != []) == (status == 0)


@pytest.mark.parametrize("kw,status", [
    (dict(), 0), (dict(R=7), 1), (dict(R=136), 1), (dict(D=12, R=12), 2), (dict(D=264, R=264), 2),
    (dict(norm=3), 1), (dict(out=3, out_scale=0.0), 1), (dict(out=3, out_scale=0.5), 0),
    (dict(act=1), 1), (dict(tdt=2), 1), (dict(out=2), 1), (dict(q_stride=4 * 128 - 8), 1),
    (dict(q_stride=4 * 128 + 4), 2), (dict(q_stride=1 << 28), 2), (dict(eps=-1e-6), 1),
    (dict(shift=8), 2), (dict(q_out_mode=1), 0), (dict(q_out_mode=1, out=3), 1),
    (dict(q_out_mode=2), 1), (dict(T=1 << 31), 2),
], ids=lambda v: str(v))
def test_table_argument_rules(driver, kw, status):
    args = dict(T=33, Hq=4, Hk=2, D=128, R=128, inter=0)
    args.update(kw)
    ls, st = run_table(driver, args.pop("T"), args.pop("Hq"), args.pop("Hk"), args.pop("D"),
                       args.pop("R"), **args)
    assert st == status
    assert (ls != []) == (status == 0)
