"""The launch-time divisor helper (csrc/fastdiv.hpp) against plain integer
division, on the host: every divisor up to 4096 and a spread of larger
ones, each with numerators 0..70000, the values around every multiple of
the divisor near the top of the range, and 2^31 - 1."""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SRC = r"""
#include <stdio.h>
#include <stdint.h>
#define __host__
#define __device__
#include "fastdiv.hpp"
using namespace dsv4;
static int check(uint32_t n, const FastDiv& f) {
    if (fdiv(n, f) != n / f.d) { printf("FAIL n=%u d=%u got %u\n", n, f.d, fdiv(n, f)); return 1; }
    return 0;
}
int main(void) {
    uint64_t tested = 0;
    uint32_t ds[6000];
    int nd = 0;
    for (uint32_t d = 1; d <= 4096; ++d) ds[nd++] = d;
    for (uint64_t d = 4097; d < (1ull << 31); d = d * 3 / 2 + 7) ds[nd++] = (uint32_t)d;
    ds[nd++] = (1u << 31) - 1;
    for (int i = 0; i < nd; ++i) {
        const FastDiv f = make_fastdiv(ds[i]);
        for (uint32_t n = 0; n <= 70000; ++n, ++tested) if (check(n, f)) return 1;
        for (uint64_t k = ((1ull << 31) - 1) / ds[i]; k + 64 > ((1ull << 31) - 1) / ds[i] && k > 0; --k) {
            uint64_t base = k * ds[i];
            for (int e = -1; e <= 1; ++e) {
                uint64_t n = base + e;
                if (n < (1ull << 31)) { if (check((uint32_t)n, f)) return 1; ++tested; }
            }
        }
        if (check((1u << 31) - 1, f)) return 1;
    }
    printf("FASTDIV OK %llu\n", (unsigned long long)tested);
    return 0;
}
"""


def test_fastdiv_matches_integer_division(tmp_path):
    src = tmp_path / "fd.cpp"
    src.write_text(SRC)
    exe = tmp_path / "fd"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I",
                    os.path.join(ROOT, "sparse_mla_attention_block_amd", "csrc"), str(src), "-o",
                    str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "FASTDIV OK" in r.stdout, r.stdout + r.stderr
