"""The oracle's pins catch plausible mistakes: each mutation below plants one into a scratch
copy of oracle/oracle.c, builds it, and runs the CPU pin files (test_oracle_math.py,
test_oracle_formats.py, test_oracle_cam.py) against that build; at least one pin must fail.

The mutations are the mistakes an implementation of these pages could plausibly make: a wrong
rounding or exponent bias in a number format, eps outside the root, a sum for a mean, the
(1 + w) weight form, a weight indexed by head, a flipped rotation sign, a wrong pairing or table
column, swapped grid axes, a YaRN blend the wrong way round, the attention factor dropped, an
ignored token offset, V taken from K, and in the camera prologue a dropped or absolute ReLU, a
NaN-zeroing ReLU, a transposed matrix, the wrong zero-norm value, the K scale dropped or V
rectified. Every mutation keeps memory accesses in bounds. CPU only; nothing here touches a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "oracle", "oracle.c")
PINS = ["tests/test_oracle_math.py", "tests/test_oracle_formats.py", "tests/test_oracle_cam.py"]

# (name, text in oracle.c, replacement); each text occurs exactly once
MUTATIONS = [
    # number formats
    ("bf16 decode shift", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    ("f16 subnormal quantum", "else if (E == 0) v = ldexp((double)M, -24);",
     "else if (E == 0) v = ldexp((double)M, -25);"),
    ("f16 exponent bias", "else v = ldexp(1.0 + M / 1024.0, E - 15);",
     "else v = ldexp(1.0 + M / 1024.0, E - 14);"),
    ("ties away from zero", "return rint(a / quantum) * quantum;",
     "return floor(a / quantum + 0.5) * quantum;"),
    ("no subnormal floor", "if (lead < emin) lead = emin;", ";"),
    ("bf16 largest finite", "double max_finite = ldexp(255.0, 120);",
     "double max_finite = ldexp(255.0, 119);"),
    ("f16 overflow code", "if (r > 65504.0) return sign | 0x7C00;",
     "if (r > 65504.0) return sign | 0x7BFF;"),
    ("f16 mantissa scale", "int mant = (int)((r / ldexp(1.0, lead) - 1.0) * 1024.0);",
     "int mant = (int)((r / ldexp(1.0, lead) - 1.0) * 1023.0);"),
    ("e4m3 saturation limit", "if (a > 448.0) a = 448.0;", "if (a > 480.0) a = 480.0;"),
    ("e4m3 NaN code", "if (isnan(x)) return signbit(x) ? 0xFF : 0x7F;",
     "if (isnan(x)) return signbit(x) ? 0xFE : 0x7E;"),
    ("e4m3 subnormal quantum", "return (uint8_t)(sign | (int)(r / ldexp(1.0, -9)));",
     "return (uint8_t)(sign | (int)(r / ldexp(1.0, -10)));"),
    ("e4m3 exponent bias", "return (uint8_t)(sign | ((lead + 7) << 3) | mant);",
     "return (uint8_t)(sign | ((lead + 8) << 3) | mant);"),
    ("e4m3 decode bias", "else v = ldexp(1.0 + M / 8.0, E - 7);",
     "else v = ldexp(1.0 + M / 8.0, E - 8);"),
    ("e4m3 scale divides", "out[i] = oracle_e4m3_encode(x[i] * scale);",
     "out[i] = oracle_e4m3_encode(x[i] / scale);"),
    # RMSNorm
    ("eps outside the root", "return 1.0 / sqrt(sum / (double)n + eps);",
     "return 1.0 / (sqrt(sum / (double)n) + eps);"),
    ("sum instead of mean", "return 1.0 / sqrt(sum / (double)n + eps);",
     "return 1.0 / sqrt(sum + eps);"),
    ("weight as 1 + w", "x[h * D + d] = x[h * D + d] * r * act_decode(act, w[d]);",
     "x[h * D + d] = x[h * D + d] * r * (1.0 + act_decode(act, w[d]));"),
    ("per-head scale of head 0", "double r = inv_rms(x + (int64_t)h * D, D, eps);",
     "double r = inv_rms(x, D, eps);"),
    ("across-heads weight per head", "x[i] = x[i] * r * act_decode(act, w[i]);",
     "x[i] = x[i] * r * act_decode(act, w[i % D]);"),
    ("across-heads over one head", "double r = inv_rms(x, (int64_t)H * D, eps);",
     "double r = inv_rms(x, D, eps);"),
    # table-form RoPE
    ("table rotation sign a", "oh[a] = nh[a] * c - nh[b] * s;", "oh[a] = nh[a] * c + nh[b] * s;"),
    ("table rotation sign b", "oh[b] = nh[b] * c + nh[a] * s;", "oh[b] = nh[b] * c - nh[a] * s;"),
    ("half-split pairs reversed", "int a = interleaved ? 2 * i : i;",
     "int a = interleaved ? 2 * i : R / 2 - 1 - i;"),
    ("sin column reversed", "double s = table_value(sin_table, dtype, sin_row + i);",
     "double s = table_value(sin_table, dtype, sin_row + R / 2 - 1 - i);"),
    ("unrotated dims zeroed", "for (int d = 0; d < D; ++d) oh[d] = nh[d];",
     "for (int d = 0; d < D; ++d) oh[d] = 0.0 * nh[d];"),
    ("packed sin columns shifted", "(const char *)rope_table + (size_t)(rotary_dim / 2) * esize",
     "(const char *)rope_table + (size_t)(rotary_dim / 2 - 2) * esize"),
    ("Q normalised with K's weights",
     "table_token(q + t * q_stride, act_dtype, num_heads_q, D, R, interleaved, norm_mode,\n"
     "                        q_weight,",
     "table_token(q + t * q_stride, act_dtype, num_heads_q, D, R, interleaved, norm_mode,\n"
     "                        k_weight,"),
    # 3D form
    ("frame index", "pos[0] = s / ((int64_t)pph * ppw);", "pos[0] = s / ((int64_t)pph);"),
    ("height index", "pos[1] = (s / ppw) % pph;", "pos[1] = s % pph;"),
    ("width index", "pos[2] = s % ppw;", "pos[2] = (s / pph) % ppw;"),
    ("frequency exponent", "double omega = pow(base, -2.0 * j / (double)C[axis]);",
     "double omega = pow(base, -1.0 * j / (double)C[axis]);"),
    ("axes reversed", "double theta = (double)pos[axis] * omega;",
     "double theta = (double)pos[2 - axis] * omega;"),
    ("YaRN ramp width", "double rho = (j - low) / (high - low);",
     "double rho = (j - low) / (high - low + 1.0);"),
    ("YaRN multiplies by factor", "omega = (omega / factor) * rho + omega * (1.0 - rho);",
     "omega = (omega * factor) * rho + omega * (1.0 - rho);"),
    ("attention factor dropped", "*c = cos(theta) * attention_factor;", "*c = cos(theta);"),
    ("3D rotation sign", "oh[a] = nh[a] * cs_c[k] - nh[b] * cs_s[k];",
     "oh[a] = nh[a] * cs_c[k] + nh[b] * cs_s[k];"),
    ("3D NeoX partner mirrored", "int b = interleave ? 2 * k + 1 : k + D / 2;",
     "int b = interleave ? 2 * k + 1 : D - 1 - k;"),
    ("token offset ignored", "grid_position((token_offset + i) % S, pph, ppw, pos);",
     "grid_position(i % S, pph, ppw, pos);"),
    ("V taken from K", "v_out[i * Hv * D + e] = oracle_bf16_decode(src[(int64_t)(Hq + Hk) * D + e]);",
     "v_out[i * Hv * D + e] = oracle_bf16_decode(src[(int64_t)Hq * D + e]);"),
    # sums of squares
    ("signed squares", "sq += v * v;", "sq += fabs(v) * v;"),
    ("K sums read Q", "double v = oracle_bf16_decode(x[nq + i]);",
     "double v = oracle_bf16_decode(x[i]);"),
    # camera prologue
    ("camera ReLU as |x|", "if (relu) v = (v > 0.0 || isnan(v)) ? v : 0.0;",
     "if (relu) v = fabs(v);"),
    ("camera ReLU zeroes NaN", "if (relu) v = (v > 0.0 || isnan(v)) ? v : 0.0;",
     "if (relu) v = v > 0.0 ? v : 0.0;"),
    ("camera matrix transposed", "acc += (double)P[4 * i + j] * a[4 * g + j];",
     "acc += (double)P[4 * j + i] * a[4 * g + j];"),
    ("camera rotation sign", "y[2 * i] = p[2 * i] * c - p[2 * i + 1] * s;",
     "y[2 * i] = p[2 * i] * c + p[2 * i + 1] * s;"),
    ("inflation of a zero key", "return na == 0.0 ? 1.0 : np_ / na;",
     "return na == 0.0 ? 0.0 : np_ / na;"),
    ("camera V with Q's matrix",
     "cam_head(v + bn * v_stride + (int64_t)h * D, act_dtype, 0, 1.0, proj_kv + bn * 16,",
     "cam_head(v + bn * v_stride + (int64_t)h * D, act_dtype, 0, 1.0, proj_q + bn * 16,"),
    ("camera K scale dropped",
     "double infl = cam_head(k + bn * k_stride + (int64_t)h * D, act_dtype, 1, k_scale,",
     "double infl = cam_head(k + bn * k_stride + (int64_t)h * D, act_dtype, 1, 1.0,"),
    ("camera ReLU on V",
     "cam_head(v + bn * v_stride + (int64_t)h * D, act_dtype, 0, 1.0, proj_kv + bn * 16,",
     "cam_head(v + bn * v_stride + (int64_t)h * D, act_dtype, 1, 1.0, proj_kv + bn * 16,"),
]


def _run_one(mut, workdir):
    name, old, new = mut
    text = open(SOURCE).read()
    src = os.path.join(workdir, "oracle_mutant.c")
    lib = os.path.join(workdir, "liboracle_mutant.so")
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    r = subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-w", "-o", lib, src, "-lm"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        return name, "build failed: " + r.stderr[-500:]
    env = dict(os.environ, QKROPE_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PINS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, "caught" if r.returncode != 0 else "survived"


def test_every_mutation_occurs_once():
    text = open(SOURCE).read()
    for name, old, new in MUTATIONS:
        assert text.count(old) == 1, f"{name}: the mutated text occurs {text.count(old)} times"
        assert old != new


def test_every_planted_mistake_fails_a_pin(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("needs gcc")
    dirs = []
    for i in range(len(MUTATIONS)):
        d = tmp_path / f"m{i}"
        d.mkdir()
        dirs.append(str(d))
    control = tmp_path / "control"
    control.mkdir()
    workers = min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        # the control is the unmutated source built the same way: it must pass every pin, so a
        # failure of a mutant is the planted mistake's, not the harness's
        ctl = ex.submit(_run_one, ("control", "", ""), str(control))
        results = list(ex.map(_run_one, MUTATIONS, dirs))
    assert ctl.result() == ("control", "survived"), ctl.result()
    bad = [(n, r) for n, r in results if r != "caught"]
    assert not bad, f"{len(bad)} of {len(MUTATIONS)} planted mistakes not caught: {bad}"
