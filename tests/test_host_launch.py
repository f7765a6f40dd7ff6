"""The host side of the C ABI (qkrope_api.cpp) on the CPU: launch shapes and launch loops.

A small C++ program compiles the library's own host source with the kernel launchers and the
few HIP runtime calls it makes replaced by stubs that record each launch (its kernel key,
launch shape, token range and input offset) instead of running it. The entry points then run
unchanged on fake, never-dereferenced device addresses. This pins:
  * the launch shape each named workload gets (the shapes the kernels were tuned for);
  * the region split (three workgroups per token) where it applies, and only there;
  * calls whose grid exceeds one dispatch: how many launches, their token ranges, grid sizes,
    pointer offsets and position offsets, at sizes no GPU test allocates;
  * that every address range a launch lets its kernel form lies inside one of the caller's
    tensors: the stubs model each kernel's reads and writes (token rows of every region, idle
    slots reading a row's first chunk, norm weights, table rows, the sums of a sharded call, the
    camera prologue's matrices and tables) from the launch's arguments and check them against
    the tensors the call was given. This covers regions without heads (which borrow another
    region's row and weights), launches split over token ranges and two-token workgroups, with
    no GPU. The same program also runs under AddressSanitizer and UndefinedBehaviorSanitizer.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "qk_rmsnorm_rope_amd", "csrc")

DRIVER = r"""
#include "qkrope_api.cpp"
#include "qkrope_api_cam.cpp"

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

// ---- the caller's tensors, and the ranges a launch lets its kernel touch -------------------
struct Span { uintptr_t lo, hi; };
static std::vector<Span> g_spans;
static void reg(const void *p, long long bytes)
{
    if (p && bytes > 0) g_spans.push_back({reinterpret_cast<uintptr_t>(p),
                                           reinterpret_cast<uintptr_t>(p) + (uintptr_t)bytes});
}
// [p, p + bytes) must lie inside one caller tensor
static void need(const void *p, long long bytes, const char *what)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p), hi = lo + (uintptr_t)bytes;
    for (const Span &s : g_spans)
        if (lo >= s.lo && hi <= s.hi) return;
    std::printf("OOB %s at %#llx + %lld bytes\n", what, (unsigned long long)lo, bytes);
}

// The prologue kernel's accesses (qkrope_kernel_impl.h), per launch of T tokens: every slot
// reads 16 bytes of its region's token row at its head's chunk (an idle slot, or a region
// without heads, the row's first chunk); stores go to the region's output rows; per-head
// weights are read at a chunk of [head_dim], across-heads weights at [heads * head_dim] (the
// first chunk for a region without heads); table rows at columns below rotary_dim / 2; a
// sharded call's sums at [T, 2].
static void check_prologue(const qkrope::KernelKey &k, const qkrope::KernelArgs &a)
{
    const bool is3d = k.src == qkrope::kSrc3D;
    const int nreg = is3d ? 3 : 2;
    const long long T = a.num_tokens, D = a.head_dim;
    const int esize = k.fp8 ? 1 : 2;
    static const char *in_names[3] = {"load q", "load k", "load v"};
    static const char *out_names[3] = {"store q", "store k", "store v"};
    for (int r = 0; r < nreg; ++r) {
        const long long width = a.heads[r] > 0 ? a.heads[r] * D : 8;
        need(a.in[r], ((T - 1) * a.in_stride[r] + width) * 2, in_names[r]);
        if (a.heads[r] > 0)
            need(a.out[r], ((T - 1) * a.out_stride[r] + a.heads[r] * D) * esize, out_names[r]);
    }
    if (k.norm == qkrope::kNormPerHead) {
        need(a.weight[0], D * 2, "q weight");
        need(a.weight[1], D * 2, "k weight");
    } else if (k.norm == qkrope::kNormAcross || k.norm == qkrope::kNormAcrossExt) {
        need(a.weight[0], a.heads[0] > 0 ? a.heads[0] * D * 2 : 16, "q weight");
        need(a.weight[1], a.heads[1] > 0 ? a.heads[1] * D * 2 : 16, "k weight");
    }
    if (!is3d && a.rotary_dim > 0) {
        const long long ts = k.src == qkrope::kSrcTableF32 ? 4 : 2, half = a.rotary_dim / 2;
        need(a.table_cos, ((T - 1) * a.cos_stride + half) * ts, "cos table");
        need(a.table_sin, ((T - 1) * a.sin_stride + half) * ts, "sin table");
    }
    if (a.sumsq_in) need(a.sumsq_in, T * 8, "sums in");
}

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
                "pairing=%d norm=%d fp8=%d ntok=%lld toff=%u in0=%llu xcd=%u xlg=%u xfull=%u dev=%u\n",
                kind, s.threads, s.slots, (int)s.slot_uniform, s.tpw, (int)s.split,
                (long long)s.blocks, k.head_dim_tpl, k.pairing, k.norm, (int)k.fp8,
                (long long)a.num_tokens, a.token_offset,
                (unsigned long long)(reinterpret_cast<uintptr_t>(a.in[0]) - g_base), a.xcd_group,
                a.xcd_lg, a.xcd_full, a.store_device);
    check_prologue(k, a);
    return hipSuccess;
}
#define STUB(name) \
    hipError_t qkrope::name(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t) \
    { return rec(#name, k, s, a); }
STUB(launch_3d_d64) STUB(launch_3d_d128) STUB(launch_3d_d256)
STUB(launch_table_interleaved_bf16) STUB(launch_table_halfsplit_bf16)
STUB(launch_table_interleaved_f16) STUB(launch_table_halfsplit_f16)
STUB(launch_table_halfsplit_any_bf16) STUB(launch_table_halfsplit_any_f16)
hipError_t qkrope::launch_sumsq(const SumsqArgs &a, int64_t tokens, int threads, hipStream_t)
{
    std::printf("launch sumsq threads=%d tokens=%lld\n", threads, (long long)tokens);
    const long long chunks = a.q_chunks + a.k_chunks;      // 16-byte chunks read per token
    if (chunks > 0) need(a.qkv, ((tokens - 1) * a.row + chunks * 8) * 2, "sums load");
    need(a.out, tokens * 8, "sums store");
    return hipSuccess;
}

hipError_t qkrope::launch_cam(const CamArgs &a, int act, int cpl, int64_t blocks, int lds_bytes,
                              hipStream_t)
{
    std::printf("launch cam act=%d cpl=%d lanes=%d hpg=%d groups=%d tiles=%d tiles_padded=%d "
                "xcd=%u blocks=%lld lds=%d row_chunks=%d vec=%d pitch=%lld\n",
                act, cpl, a.lanes_per_token, a.heads_per_group, a.groups, a.tiles, a.tiles_padded,
                a.xcd_group, (long long)blocks, lds_bytes, a.row_chunks, a.vec_store,
                (long long)a.out_row_stride);
    // qkrope_kernels_cam.hip: token rows of q, k, v; one 4x4 fp32 matrix per (b, n) each; table
    // rows [N, D/2]; output rows (b, h, d) of N values, out_row_stride apart; inflation [B, H, N]
    const long long BN = (long long)a.batch * a.num_tokens, D = a.head_dim, H = a.heads;
    const long long rows = (long long)a.batch * H * D;
    for (int r = 0; r < 3; ++r) {
        need(a.in[r], ((BN - 1) * a.in_stride[r] + H * D) * 2, "cam load");
        need(a.out[r], ((rows - 1) * a.out_row_stride + a.num_tokens) * 2, "cam store");
    }
    need(a.proj[0], BN * 64, "proj_q");
    need(a.proj[1], BN * 64, "proj_kv");
    need(a.cos_table, a.num_tokens * (D / 2) * 4, "cam cos");
    need(a.sin_table, a.num_tokens * (D / 2) * 4, "cam sin");
    if (a.inflation) need(a.inflation, BN * H * 4, "inflation");
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
    // QKROPE_TEST_SHRINK=n: the first input is registered n bytes short (a check of the checker)
    const long long shrink = std::getenv("QKROPE_TEST_SHRINK") ? std::atoll(std::getenv("QKROPE_TEST_SHRINK")) : 0;
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
        const long long es = I(13) ? 1 : 2;
        reg(qkv, T * (I(7) + I(8) + I(9)) * D * 2 - shrink);
        reg(qo, T * I(7) * D * es);
        reg(at(2), T * I(8) * D * es);
        reg(at(3), T * I(9) * D * es);
        reg(at(4), I(7) * D * 2);
        reg(at(5), I(8) * D * 2);
        if (sums) reg(at(6), T * 8);
        st = qkrope_run_3d_sharded(h, qkv, at(4), at(5), T, I(14), sums ? (const float *)at(6) : nullptr,
                                   (I(7) ? I(7) : 1) * D, (I(8) ? I(8) : 1) * D, (int)I(1), (int)I(2), (int)I(3), (int)I(4),
                                   (int)I(5), (int)I(6), (int)I(7), (int)I(8), (int)I(9), D, v[16],
                                   v[17], (int)I(11), v[18], v[19], v[20], v[21], (int)I(12),
                                   (int)I(13), v[22], v[23], qo, at(2), at(3), nullptr);
    } else if (!std::strcmp(form, "sumsq")) {
        // T Hq Hk Hv D
        const long long T = I(0);
        const int D = (int)I(4);
        reg(at(0), T * (I(1) + I(2) + I(3)) * D * 2 - shrink);
        reg(at(6), T * 8);
        st = qkrope_sumsq_3d(h, at(0), T, (int)I(1), (int)I(2), (int)I(3), D, (float *)at(6),
                             nullptr);
    } else if (!std::strcmp(form, "cam")) {
        // B N H D act [out_row_stride, 0: N]
        const long long B = I(0), N = I(1);
        const int H = (int)I(2), D = (int)I(3);
        const long long s = (long long)H * D, rp = I(5) ? I(5) : N;
        const long long out_bytes = B * s > 0 ? ((B * s - 1) * (rp > N ? rp : N) + N) * 2 : 0;
        for (int i = 0; i < 3; ++i) reg(at(i), B * N * s * 2 - (i == 0 ? shrink : 0));
        reg(at(3), B * N * 64);
        reg(at(4), B * N * 64);
        reg(at(5), N * (D / 2) * 4);
        reg(at(6), N * (D / 2) * 4);
        for (int i = 7; i < 10; ++i) reg(at(i), out_bytes);
        reg(at(10), B * H * N * 4);
        st = qkrope_cam_prep(h, at(0), at(1), at(2), (int)I(4), (const float *)at(3),
                             (const float *)at(4), (const float *)at(5), (const float *)at(6),
                             0.5f, B, N, H, D, s, s, s, at(7), at(8), at(9), rp, (float *)at(10),
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
        const long long os = I(8) == 3 ? 1 : 2, ts = I(9) == 1 ? 4 : 2;
        const long long wl = I(6) == 2 ? 0 : D;            // per-head weights [D]
        reg(q, ((T - 1) * qs + (long long)Hq * D) * 2 - shrink);
        reg(at(1), T * Hk * D * 2);
        reg(at(2), T * (R / 2) * ts);
        reg(at(3), T * (R / 2) * ts);
        if (I(14) == 0) reg(qo, ((T - 1) * qs + (long long)Hq * D) * os);
        reg(at(5), T * Hk * D * os);
        reg(at(6), (wl ? wl : (long long)Hq * D) * 2);
        reg(at(7), (wl ? wl : (long long)Hk * D) * 2);
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


def run(driver, *args, shrink=0, allow_oob=False):
    """The recorded launches (dicts of their fields) and the call's status. Fails if any launch
    lets its kernel touch memory outside the caller's tensors (unless allow_oob)."""
    env = dict(os.environ, QKROPE_TEST_SHRINK=str(shrink)) if shrink else None
    out = subprocess.run([driver, *map(str, args)], capture_output=True, text=True, timeout=60,
                         check=True, env=env).stdout.splitlines()
    oob = [l for l in out if l.startswith("OOB ")]
    if oob and not allow_oob:
        raise AssertionError(f"{args}: out-of-tensor ranges: {oob[:4]}")
    if allow_oob:
        return oob
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
    assert l["blocks"] == 36960 // 2 and l["xcd"] == 16
    # 122880 x 3x16 x 256, no norm: one region of one token per workgroup (three per token)
    (l,), st = run_3d(driver, 122880, (32, 48, 80), (64, 96, 96), (16, 16, 16), 256, norm=0)
    assert st == 0 and (l["threads"], l["split"], l["norm"]) == (512, 1, 0)
    assert l["blocks"] == 3 * 122880 and l["xcd"] == 64


@pytest.mark.parametrize("norm,fp8,heads", [(1, 0, (16, 16, 16)), (0, 1, (16, 16, 16)),
                                            (0, 0, (4, 4, 4))])
def test_region_split_only_without_norm_for_16_bit_outputs_and_wide_rows(driver, norm, fp8,
                                                                         heads):
    (l,), st = run_3d(driver, 1536, (4, 4, 96), (64, 96, 96), heads, 256, norm=norm, fp8=fp8)
    assert st == 0 and l["split"] == 0 and l["blocks"] == 1536 // l["tpw"]


def test_xcd_renumbering_parameters_match_the_run_length(driver):
    # the kernel renumbers blocks below xfull (whole runs of 8 * 2^xlg blocks) branch-free;
    # the host derives both from the run length G = xcd and the launch's grid
    launches = [run_3d(driver, 15360, (16, 24, 40), (16, 56, 56), (32, 32, 32), 128)[0][0],
                run_3d(driver, 36960, (20, 33, 28), (16, 24, 24), (20, 20, 20), 64, interleave=0,
                       fp8=1)[0][0],
                run_3d(driver, 122880, (32, 48, 80), (64, 96, 96), (16, 16, 16), 256,
                       norm=0)[0][0],
                run_table(driver, 4096, 24, 24, 128, 128, tdt=0)[0][0],
                run_table(driver, 100, 2, 2, 128, 128, tdt=0)[0][0]]     # 100 blocks: plain order
    for l in launches:
        G = l["xcd"]
        if G == 0:
            assert l["xlg"] == 0 and l["xfull"] == 0 and l["blocks"] < 128
            continue
        assert 1 << l["xlg"] == G
        assert l["xfull"] == l["blocks"] // (8 * G) * (8 * G) and l["xfull"] > 0
        # the renumbering (the kernel's shifts and masks): a permutation of the grid in which
        # the hardware's XCD b % 8 gets runs of G consecutive blocks
        lg, full = l["xlg"], l["xfull"]
        b = np.arange(l["blocks"], dtype=np.int64)
        j, x = b >> 3, b & 7
        r = ((j >> lg) << (lg + 3)) + (x << lg) + (j & ((1 << lg) - 1))
        r = np.where(b < full, r, b)
        assert np.array_equal(np.sort(r), b)
        # hardware block 8j + x goes to XCD x: [run][position j in the run][XCD x]
        runs = r[: full].reshape(-1, G, 8)
        assert (np.diff(runs, axis=1) == 1).all()
    assert [l["xcd"] for l in launches] == [16, 16, 64, 16, 0]


def test_store_scope_follows_the_bytes_a_launch_writes(driver):
    # device-scope stores once a launch writes at least 2^27 bytes
    cases_3d = [((32, 32, 32), 128, 15360, 0, 1),     # 15360 x 3x32 x 128: 377 MB
                ((8, 8, 8), 128, 15360, 0, 0),        # one rank of 4 head shards: 94 MB
                ((20, 20, 20), 64, 36960, 1, 1)]      # 2 x 18480 x 3x20 x 64, E4M3: 142 MB
    for heads, D, T, fp8, dev in cases_3d:
        grid = (20, 33, 28) if T == 36960 else (16, 24, 40)
        ch = (16, 24, 24) if D == 64 else (16, 56, 56)
        (l,), st = run_3d(driver, T, grid, ch, heads, D, interleave=1 - fp8, fp8=fp8)
        assert st == 0 and l["dev"] == dev, (heads, D, T)
    for T, dev in [(4096, 0), (32768, 1)]:                  # 2x24 x 128 tables: 50 / 403 MB
        (l,), st = run_table(driver, T, 24, 24, 128, 128, tdt=0)
        assert st == 0 and l["dev"] == dev, T
    # the threshold itself: 4096 bytes a token (2x8 x 128 bf16), 2^15 tokens write 2^27 bytes
    for T, dev in [(32767, 0), (32768, 1)]:
        (l,), st = run_table(driver, T, 8, 8, 128, 128, tdt=0)
        assert st == 0 and l["dev"] == dev, T
    (l,), st = run_table(driver, 2 * 32768, 8, 8, 128, 128, tdt=0, out=3)   # E4M3: a byte each
    assert st == 0 and l["dev"] == 1 and l["fp8"] == 1


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
    # store scope and XCD runs are chosen per launch: the first writes far more than 2^27
    # bytes, the second 3001 tokens x 80 heads x 128 x 2 bytes (61 MB)
    assert (a["dev"], b["dev"]) == (1, 0)
    assert a["xcd"] == b["xcd"] == 64
    assert (a["xfull"], b["xfull"]) == (a["blocks"] // 512 * 512, b["blocks"] // 512 * 512)


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
    # 288 tiles: eighths without padding
    (l,), st = run(driver, "cam", 2, 18432, 20, 64, 0)
    assert st == 0 and (l["tiles_padded"], l["xcd"], l["blocks"]) == (288, 36, 2 * 10 * 288)
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
    # padded output rows: the pitch reaches the kernel; 16-byte stores need a multiple of 8, and
    # every store stays inside the B*H*D rows of N values (run() checks the ranges)
    (l,), st = run(driver, "cam", 2, 18480, 20, 64, 0, 18496)
    assert st == 0 and (l["pitch"], l["vec"]) == (18496, 1)
    (l,), st = run(driver, "cam", 2, 200, 3, 64, 0, 203)
    assert st == 0 and (l["pitch"], l["vec"]) == (203, 0)
    (l,), st = run(driver, "cam", 1, 301, 2, 40, 0, 304)
    assert st == 0 and (l["pitch"], l["vec"]) == (304, 1)     # N % 8 != 0, rows still aligned


@pytest.mark.parametrize("pitch,status", [(199, 1), (1, 1), (1 << 31, 2), (200, 0), (256, 0)])
def test_camera_prologue_row_pitch_rules(driver, pitch, status):
    """out_row_stride: below num_tokens is invalid, 2^31 and past unsupported; nothing launches
    unless the call is accepted."""
    ls, st = run(driver, "cam", 2, 200, 3, 64, 0, pitch)
    assert st == status and len(ls) == (1 if status == 0 else 0)


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
    # seq_len = ppf*pph*ppw must be < 2^31 (32-bit position division): pph*ppw = 2^32 once
    # truncated to 0 (a division by zero on the host), 46341^2 = 2^31 + 4281 gave a shift of 32
    # in the kernel; products past int64 are refused as well
    (dict(grid=(1, 65536, 65536)), 2), (dict(grid=(1, 46341, 46341)), 2),
    (dict(grid=(46341, 46341, 1)), 2), (dict(grid=(2147483647, 2147483647, 2147483647)), 2),
    (dict(grid=(1, 46340, 46340)), 0), (dict(grid=(2, 1 << 15, (1 << 15) - 1)), 0),
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


# --- every address a launch lets its kernel form lies in a caller's tensor ----------------------
# (run() checks this for every launch of every test above; these cases aim at the edges)

def test_range_check_catches_a_tensor_one_chunk_short(driver):
    """The checker is not vacuous: registering the input 16 bytes short is caught."""
    oob = run(driver, "3d", 120, 2, 3, 4, 32, 48, 48, 4, 2, 2, 128, 1, 1, 0, 0, 0, 1e-6, 1e4,
              1.0, 0.0, 0.0, 1.0, 1.0, 1.0, 0, 0, shrink=16, allow_oob=True)
    assert oob and oob[0].startswith("OOB load v")
    oob = run(driver, "table", 33, 4, 2, 128, 128, 0, 1, 0, 0, 1, 0, 1e-6, 1.0, 0, 0,
              shrink=16, allow_oob=True)
    assert oob and oob[0].startswith("OOB load q")
    assert run(driver, "cam", 2, 130, 3, 64, 0, shrink=16, allow_oob=True)[0].startswith("OOB cam")
    assert run(driver, "sumsq", 50, 4, 4, 0, 64, shrink=16, allow_oob=True)


@pytest.mark.parametrize("Hq,Hk,norm", [(0, 3, 1), (0, 3, 2), (3, 0, 1), (3, 0, 2), (0, 2, 0),
                                        (5, 0, 0)])
def test_table_regions_without_heads_stay_in_bounds(driver, Hq, Hk, norm):
    """A region without heads (NULL-able pointers) borrows the other region's row and weights."""
    for inter in (0, 1):
        (l,), st = run_table(driver, 37, Hq, Hk, 128, 96, inter=inter, norm=norm)
        assert st == 0


@pytest.mark.parametrize("heads,norm,fp8,sums", [
    ((4, 0, 2), 1, 0, 0), ((4, 2, 0), 1, 1, 0), ((0, 3, 3), 1, 0, 0), ((0, 0, 5), 0, 0, 0),
    ((2, 2, 0), 1, 0, 1), ((0, 4, 1), 1, 1, 1), ((6, 0, 0), 0, 1, 0),
])
def test_3d_regions_without_heads_stay_in_bounds(driver, heads, norm, fp8, sums):
    (l,), st = run_3d(driver, 24, (2, 3, 4), (32, 48, 48), heads, 128, norm=norm, fp8=fp8,
                      sums=sums)
    assert st == 0


def test_two_token_workgroups_with_an_odd_token_count(driver):
    # 160 lanes a token, two tokens per workgroup: the last workgroup's missing second token
    # re-reads the first one's row and stores nothing
    (l,), st = run_3d(driver, 15, (1, 3, 5), (16, 24, 24), (20, 20, 20), 64, interleave=0, fp8=1)
    assert st == 0 and l["tpw"] == 2 and l["blocks"] == 8


def test_sums_kernel_ranges_and_launch_loop(driver):
    per = ((1 << 32) - 1) // 64          # one head of 64 in Q and K: 64-lane workgroups
    ls, st = run(driver, "sumsq", per + 7, 1, 1, 1, 64)
    assert st == 0 and [l["tokens"] for l in ls] == [per, 7]
    ls, st = run(driver, "sumsq", 300, 0, 0, 3, 64)             # no Q or K heads: zeros written
    assert st == 0 and len(ls) == 1
    ls, st = run(driver, "sumsq", 64, 48, 48, 48, 128)          # rows wider than one workgroup
    assert st == 0 and ls[0]["threads"] == 768


def test_two_tokens_per_workgroup_only_for_strides_below_2_24_bytes(driver):
    # 20 heads of 64 in each of Q and K: 160 lanes a token, two tokens per workgroup; the kernel
    # forms the second token's offsets with 24-bit multiplies, so wide strides take one token
    (l,), st = run_table(driver, 33, 20, 20, 64, 64)
    assert st == 0 and l["tpw"] == 2
    (l,), st = run_table(driver, 33, 20, 20, 64, 64, q_stride=(1 << 23) - 8)
    assert st == 0 and l["tpw"] == 2
    (l,), st = run_table(driver, 33, 20, 20, 64, 64, q_stride=1 << 23)
    assert st == 0 and l["tpw"] == 1 and l["blocks"] == 33
