"""The host's magic divisors (qkrope_host.h, make_fast_div) against exact integer division.

The kernels split a token index into (sequence, frame, row, column) and a block index into
(batch, head group, tile) with q = (mulhi(n, m) + n) >> l for n < 2^31. A small C++ program
built from the library's own host header checks that q equals n / d for every divisor up to
4096, powers of two and their neighbours, and random divisors up to 2^31 - 1, each over edge
numerators (0, d - 1, d, multiples of d and their neighbours, 2^31 - 1) and random ones.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "qk_rmsnorm_rope_amd", "csrc")

CHECKER = r"""
#include "qkrope_internal.h"
#include "qkrope_host.h"
#include <cstdint>
#include <cstdio>
#include <vector>

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd31() {                       // splitmix64, top 31 bits
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 33);
}

static int check(uint32_t d) {
    const qkrope::FastDiv f = qkrope::host::make_fast_div(d);
    const uint32_t top = 0x7FFFFFFFu;
    std::vector<uint32_t> ns = {0u, 1u, d - 1, d, d + 1, top, top - 1, top / d * d, top / d * d - 1};
    for (uint32_t k = 2; k < 6; ++k)
        if ((uint64_t)k * d <= top) { ns.push_back(k * d - 1); ns.push_back(k * d); }
    for (int i = 0; i < 200; ++i) ns.push_back(rnd31());
    const uint64_t span = 64ull * d < top ? 64ull * d : top;   // small multiples of d
    for (int i = 0; i < 50; ++i) ns.push_back((uint32_t)(rnd31() % span));
    for (uint32_t n : ns) {
        if (n > top) continue;
        const uint32_t hi = (uint32_t)(((uint64_t)n * f.m) >> 32);
        const uint32_t q = (hi + n) >> f.l;
        if (q != n / d) {
            std::printf("d=%u n=%u: got %u, want %u (m=%u l=%u)\n", d, n, q, n / d, f.m, f.l);
            return 1;
        }
    }
    return 0;
}

int main() {
    long count = 0;
    for (uint32_t d = 1; d <= 4096; ++d, ++count)
        if (check(d)) return 1;
    for (uint32_t s = 12; s <= 30; ++s)
        for (int64_t e = -2; e <= 2; ++e, ++count)
            if (check((uint32_t)((1ll << s) + e))) return 1;
    if (check(0x7FFFFFFFu)) return 1;
    for (int i = 0; i < 20000; ++i, ++count) {
        const uint32_t d = rnd31();
        if (d && check(d)) return 1;
    }
    std::printf("ok %ld divisors\n", count);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_magic_divisors_match_integer_division(tmp_path):
    src = tmp_path / "fastdiv_check.cpp"
    exe = tmp_path / "fastdiv_check"
    src.write_text(CHECKER)
    subprocess.run(["g++", "-std=c++17", "-O2", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")
