"""Host check of the kernels' workgroup-index division (csrc/grkan_fastdiv.h):
a g++-built harness compares it with true division for divisors 1 .. 2^31 on
all numerators below 2^22, the top 2^22 below 2^31, a million pseudo-random
ones and every multiple of the divisor +-1 up to 10^5 multiples."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gr_kan_rational_amd", "csrc")

HARNESS = r"""
#include "grkan_fastdiv.h"
#include <cstdio>
int main() {
    using namespace grkan;
    const unsigned ds[] = {1, 2, 3, 5, 6, 7, 8, 9, 10, 16, 17, 48, 63, 64, 65, 100, 127, 128, 129, 255,
                           256, 1000, 1023, 4096, 65535, 65536, 65537, 1u << 20, (1u << 20) + 1,
                           2147483647u, 2147483648u};
    unsigned long long bad = 0, checked = 0;
    for (unsigned d : ds) {
        const FastDiv f = make_fastdiv(d);
        auto chk = [&](unsigned n) { ++checked; if (fastdiv(n, f) != n / d) ++bad; };
        for (unsigned n = 0; n < (1u << 22); ++n) chk(n);
        for (unsigned n = (1u << 31) - (1u << 22); n < (1u << 31); ++n) chk(n);
        unsigned s = 12345;
        for (int i = 0; i < 1000000; ++i) { s = s * 1664525u + 1013904223u; chk(s >> 1); }
        for (unsigned long long k = 1; k < 100000 && k * d < (1ull << 31); ++k)
            for (int e = -1; e <= 1; ++e) {
                const unsigned long long n = k * d + e;
                if (n < (1ull << 31)) chk((unsigned)n);
            }
    }
    printf("checked %llu bad %llu\n", checked, bad);
    return bad != 0;
}
"""


def test_fastdiv_matches_division(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    src = tmp_path / "fastdiv_check.cpp"
    src.write_text(HARNESS)
    exe = tmp_path / "fastdiv_check"
    subprocess.run([gxx, "-O2", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bad 0" in r.stdout
