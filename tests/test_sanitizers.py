"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two programs, each built with g++/gcc (host code only; no device code is involved) with
-fsanitize=address,undefined and every report made fatal:
  * the library's host source (qkrope_api.cpp, qkrope_api_cam.cpp) with the recording launchers
    of test_host_launch.py, run over every entry point: the named workloads' shapes, regions
    without heads, launch loops past one grid, the camera prologue, the sums kernel, and
    argument errors (each rejected before any launch);
  * the fp64 oracle (oracle/oracle.c, compiled into a small C driver) on every entry point with
    buffers allocated to their exact sizes, so a read or write one element past a tensor is
    reported: packed and split tables of every dtype with padded strides, per-head /
    across-heads / no norm, both pairings, rotary_dim < head_dim, the 3D form with YaRN, FP8
    scales and a token offset, the sums, the camera prologue with padded rows, and every
    encoder over all its codes.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from test_host_launch import CSRC, DRIVER, ROOT

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]

# (form, args...) for the host driver: one line per call, as test_host_launch.py runs them
HOST_CALLS = [
    # 3D: T ppf pph ppw cf ch cw Hq Hk Hv D interleave norm fp8 offset sums eps base factor low
    #     high af oqs vqs shift q_out_mode
    ["3d", 15360, 16, 24, 40, 16, 56, 56, 32, 32, 32, 128, 1, 1, 0, 0, 0, 1e-6, 1e4, 1, 0, 0, 1,
     1, 1, 0, 0],
    ["3d", 36960, 20, 33, 28, 16, 24, 24, 20, 20, 20, 64, 0, 1, 1, 0, 0, 1e-6, 1e4, 1, 0, 0, 1,
     0.5, 0.25, 0, 0],
    ["3d", 122880, 32, 48, 80, 64, 96, 96, 16, 16, 16, 256, 1, 0, 0, 0, 0, 1e-6, 1e4, 4, 1, 32,
     1.1386, 1, 1, 0, 0],
    ["3d", 24, 2, 3, 4, 32, 48, 48, 0, 3, 3, 128, 1, 1, 0, 5, 1, 1e-6, 1e4, 1, 0, 0, 1, 1, 1, 0,
     0],
    ["3d", 2 * (((1 << 32) - 1) // 64) + 5, 1, 1, 5, 16, 24, 24, 1, 1, 1, 64, 1, 1, 0, 3, 1, 1e-6,
     1e4, 1, 0, 0, 1, 1, 1, 0, 0],
    ["3d", 24, 1, 65536, 65536, 32, 48, 48, 2, 2, 2, 128, 1, 1, 0, 0, 0, 1e-6, 1e4, 1, 0, 0, 1,
     1, 1, 0, 0],                                                    # seq_len >= 2^31: refused
    ["3d", 24, 2, 3, 4, 32, 48, 48, 2, 2, 2, 128, 1, 1, 0, 0, 0, 1e-6, 1e4, 1, 0, 0, 1, 1, 1, 8,
     0],                                                             # misaligned: refused
    # table: T Hq Hk D R interleaved norm act out tdt q_stride eps out_scale shift q_out_mode
    ["table", 4096, 24, 24, 128, 128, 1, 1, 0, 0, 0, 0, 1e-6, 1, 0, 0],
    ["table", 256, 4, 4, 128, 96, 0, 1, 0, 0, 1, 0, 1e-6, 1, 0, 0],
    ["table", 37, 0, 3, 128, 72, 0, 2, 1, 1, 2, 0, 1e-6, 1, 0, 0],
    ["table", 33, 4, 0, 128, 128, 1, 2, 0, 3, 1, 1024, 1e-6, 0.5, 0, 0],
    ["table", 33, 4, 2, 128, 128, 0, 1, 0, 0, 1, 0, 1e-6, 1, 0, 1],   # in place
    ["table", 33, 4, 2, 128, 7, 0, 1, 0, 0, 1, 0, 1e-6, 1, 0, 0],     # odd rotary_dim: refused
    ["table", ((1 << 32) - 1) // 64 + 9, 1, 1, 8, 8, 1, 1, 0, 0, 1, 0, 1e-6, 1, 0, 0],
    # camera prologue: B N H D act
    ["cam", 2, 18480, 20, 64, 0],
    ["cam", 1, 301, 2, 40, 2],
    ["cam", 1, 1000, 3, 128, 0],
    ["cam", 1, 1 << 29, 1, 64, 0],                                   # past one grid: refused
    # sums: T Hq Hk Hv D
    ["sumsq", 300, 8, 8, 8, 128],
    ["sumsq", 64, 48, 48, 48, 128],
    ["sumsq", 17, 0, 0, 2, 64],
]


def _sanitizer_env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def _check_clean(r, what):
    bad = [l for l in (r.stdout + r.stderr).splitlines()
           if "runtime error" in l or "AddressSanitizer" in l or "LeakSanitizer" in l]
    assert r.returncode == 0 and not bad, f"{what}: rc {r.returncode}\n" + \
        "\n".join(bad[:10]) + "\n" + r.stderr[-3000:]


@pytest.fixture(scope="module")
def tools():
    if shutil.which("g++") is None or shutil.which("gcc") is None or \
            not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs gcc, g++ and the ROCm headers")


def test_host_source_under_sanitizers(tools, tmp_path):
    src, exe = tmp_path / "launch_san.cpp", tmp_path / "launch_san"
    src.write_text(DRIVER)
    subprocess.run(["g++", "-std=c++17", "-w", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True, capture_output=True, text=True)
    env = _sanitizer_env()
    for call in HOST_CALLS:
        r = subprocess.run([str(exe), *map(str, call)], capture_output=True, text=True,
                           timeout=120, env=env)
        _check_clean(r, " ".join(map(str, call)))
        assert not any(l.startswith("OOB ") for l in r.stdout.splitlines()), call
        assert r.stdout.splitlines()[-1].startswith("status "), call


ORACLE_DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_run_table(const uint16_t *, const uint16_t *, const uint16_t *, const uint16_t *,
                     const void *, int, double, int64_t, int, int, int, int, int, int, int64_t,
                     int64_t, int64_t, double *, double *);
int oracle_run_table_split(const uint16_t *, const uint16_t *, const uint16_t *,
                           const uint16_t *, int, const void *, const void *, int, double,
                           int64_t, int, int, int, int, int, int, int64_t, int64_t, int64_t,
                           int64_t, double *, double *);
int oracle_run_3d(const uint16_t *, const uint16_t *, const uint16_t *, int64_t, int64_t, int,
                  int, int, int, int, int, int, int, int, int, double, double, int, double,
                  double, double, double, int, double *, double *, double *);
int oracle_sumsq_3d(const uint16_t *, int64_t, int, int, int, int, double *);
int oracle_cam_prep(const uint16_t *, const uint16_t *, const uint16_t *, int, const float *,
                    const float *, const float *, const float *, double, int64_t, int64_t, int,
                    int, int64_t, int64_t, int64_t, double *, double *, double *, double *);
uint16_t oracle_bf16_encode(double);
double oracle_bf16_decode(uint16_t);
uint16_t oracle_f16_encode(double);
double oracle_f16_decode(uint16_t);
uint8_t oracle_e4m3_encode(double);
double oracle_e4m3_decode(uint8_t);
void oracle_encode_bf16_array(const double *, int64_t, uint16_t *);
void oracle_encode_f16_array(const double *, int64_t, uint16_t *);
void oracle_quantize_e4m3_array(const double *, int64_t, double, uint8_t *);

static uint32_t g_state = 12345u;
static uint16_t act_value(int f16)        /* a small 16-bit activation, magnitude < 4 */
{
    g_state = g_state * 1664525u + 1013904223u;
    const double x = ((double)(g_state >> 8) / 16777216.0 - 0.5) * 6.0;
    return f16 ? oracle_f16_encode(x) : oracle_bf16_encode(x);
}
static uint16_t *acts(int64_t n, int f16)
{
    uint16_t *p = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) p[i] = act_value(f16);
    return p;
}
static void *table(int64_t n, int dtype)  /* 0 bf16, 1 f32, 2 f64, 3 f16: values in [-1, 1] */
{
    const size_t es = dtype == 2 ? 8 : dtype == 1 ? 4 : 2;
    unsigned char *p = (unsigned char *)malloc(es * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) {
        const double x = (double)((i * 37) % 201) / 100.0 - 1.0;
        if (dtype == 2) ((double *)p)[i] = x;
        else if (dtype == 1) ((float *)p)[i] = (float)x;
        else ((uint16_t *)p)[i] = dtype == 3 ? oracle_f16_encode(x) : oracle_bf16_encode(x);
    }
    return p;
}
static double *out(int64_t n) { return (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1)); }
#define CHECK(call) do { int rc_ = (call); if (rc_) { printf("FAIL %s -> %d\n", #call, rc_); return 1; } } while (0)

static int table_case(int64_t T, int Hq, int Hk, int D, int R, int inter, int norm, int f16,
                      int tdt, int64_t pad, int split)
{
    const int64_t qs = (int64_t)Hq * D + pad, ks = (int64_t)Hk * D + pad;
    uint16_t *q = acts((T - 1) * qs + (int64_t)Hq * D, f16), *k = acts((T - 1) * ks + (int64_t)Hk * D, f16);
    const int64_t wq = norm == 2 ? (int64_t)Hq * D : D, wk = norm == 2 ? (int64_t)Hk * D : D;
    uint16_t *w1 = acts(wq, f16), *w2 = acts(wk, f16);
    double *qo = out(T * Hq * D), *ko = out(T * Hk * D);
    if (split) {
        const int64_t cs = R / 2 + pad, ss = R / 2 + 2 * pad;
        void *c = table((T - 1) * cs + R / 2, tdt), *s = table((T - 1) * ss + R / 2, tdt);
        CHECK(oracle_run_table_split(q, k, w1, w2, f16, c, s, tdt, 1e-6, T, Hq, Hk, D, R, inter,
                                     norm, qs, ks, cs, ss, qo, ko));
        free(c); free(s);
    } else {
        const int64_t ts = R + pad;
        void *t = table((T - 1) * ts + R, tdt);
        CHECK(oracle_run_table(q, k, w1, w2, t, tdt, 1e-6, T, Hq, Hk, D, R, inter, norm, qs, ks,
                               ts, qo, ko));
        free(t);
    }
    free(q); free(k); free(w1); free(w2); free(qo); free(ko);
    return 0;
}

static int rope3d_case(int64_t T, int64_t off, int f, int h, int w, int cf, int ch, int cw,
                       int Hq, int Hk, int Hv, int D, int inter, double factor, int norm)
{
    const int64_t row = (int64_t)(Hq + Hk + Hv) * D;
    uint16_t *x = acts(T * row, 0), *w1 = acts((int64_t)Hq * D, 0), *w2 = acts((int64_t)Hk * D, 0);
    double *qo = out(T * Hq * D), *ko = out(T * Hk * D), *vo = out(T * Hv * D), *ss = out(2 * T);
    const double af = factor == 1.0 ? 1.0 : 1.1386;
    CHECK(oracle_run_3d(x, w1, w2, T, off, f, h, w, cf, ch, cw, Hq, Hk, Hv, D, 1e-6, 1e4, inter,
                        factor, 1.0, 32.0, af, norm, qo, ko, vo));
    CHECK(oracle_sumsq_3d(x, T, Hq, Hk, Hv, D, ss));
    uint8_t *codes = (uint8_t *)malloc((size_t)(T * Hq * D));
    oracle_quantize_e4m3_array(qo, T * Hq * D, 0.5, codes);
    uint16_t *bits = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(T * Hv * D + 1));
    oracle_encode_bf16_array(vo, T * Hv * D, bits);
    oracle_encode_f16_array(vo, T * Hv * D, bits);
    free(codes); free(bits);
    free(x); free(w1); free(w2); free(qo); free(ko); free(vo); free(ss);
    return 0;
}

static int cam_case(int64_t B, int64_t N, int H, int D, int f16, int64_t pad)
{
    const int64_t st = (int64_t)H * D + pad, rows = B * N;
    uint16_t *q = acts((rows - 1) * st + (int64_t)H * D, f16);
    uint16_t *k = acts((rows - 1) * st + (int64_t)H * D, f16);
    uint16_t *v = acts((rows - 1) * st + (int64_t)H * D, f16);
    float *pq = (float *)table(rows * 16, 1), *pk = (float *)table(rows * 16, 1);
    float *c = (float *)table(N * (D / 2), 1), *s = (float *)table(N * (D / 2), 1);
    double *qo = out(rows * H * D), *ko = out(rows * H * D), *vo = out(rows * H * D);
    double *infl = out(rows * H);
    CHECK(oracle_cam_prep(q, k, v, f16, pq, pk, c, s, 0.125, B, N, H, D, st, st, st, qo, ko, vo,
                          infl));
    free(q); free(k); free(v); free(pq); free(pk); free(c); free(s);
    free(qo); free(ko); free(vo); free(infl);
    return 0;
}

int main(void)
{
    /* table form: dtypes, pairings, norms, padded strides, split tables */
    if (table_case(37, 4, 2, 128, 96, 0, 1, 0, 1, 0, 0)) return 1;
    if (table_case(37, 4, 2, 128, 128, 1, 1, 0, 0, 8, 0)) return 1;
    if (table_case(19, 3, 5, 64, 40, 0, 2, 1, 3, 16, 1)) return 1;
    if (table_case(19, 3, 3, 64, 0, 1, 0, 0, 1, 0, 0)) return 1;
    if (table_case(11, 2, 2, 32, 30, 0, 1, 0, 2, 4, 1)) return 1;
    if (table_case(11, 0, 2, 32, 32, 1, 1, 1, 1, 0, 1)) return 1;
    /* 3D form */
    if (rope3d_case(24, 0, 2, 3, 4, 16, 24, 24, 3, 2, 5, 64, 1, 1.0, 1)) return 1;
    if (rope3d_case(30, 7, 1, 3, 5, 32, 48, 48, 4, 4, 4, 128, 0, 4.0, 1)) return 1;
    if (rope3d_case(12, 0, 1, 2, 2, 64, 96, 96, 2, 2, 2, 256, 1, 4.0, 0)) return 1;
    if (rope3d_case(8, 3, 2, 2, 2, 0, 0, 64, 1, 0, 1, 64, 0, 1.0, 1)) return 1;
    /* camera prologue */
    if (cam_case(2, 13, 3, 16, 0, 0)) return 1;
    if (cam_case(1, 9, 2, 64, 1, 8)) return 1;
    if (cam_case(2, 1, 1, 4, 0, 4)) return 1;
    /* encoders over every code */
    for (int c = 0; c < 65536; ++c) {
        (void)oracle_bf16_encode(oracle_bf16_decode((uint16_t)c));
        (void)oracle_f16_encode(oracle_f16_decode((uint16_t)c));
    }
    for (int c = 0; c < 256; ++c) (void)oracle_e4m3_encode(oracle_e4m3_decode((uint8_t)c));
    printf("oracle ok\n");
    return 0;
}
"""


def test_oracle_under_sanitizers(tools, tmp_path):
    src, exe = tmp_path / "oracle_san.c", tmp_path / "oracle_san"
    src.write_text(ORACLE_DRIVER)
    r = subprocess.run(["gcc", "-std=c11", "-w", *SAN, str(src),
                        os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env=_sanitizer_env())
    _check_clean(r, "oracle driver")
    assert "oracle ok" in r.stdout, r.stdout[-2000:]
