"""Host check of the kernels' sign of q(x) = b_1 + b_2 x + ... + b_n x^(n-1) when
the guard on the fp64 Q did not prove it (csrc/grkan_qsign.h): a g++-built
harness evaluates the header's routines and Python's exact rationals decide.
qsign_integer (integer Horner over the fp32 mantissas in a 256-bit window) is
what the kernels use for n >= 5, qsign_compensated (compensated Horner in fp64)
below that.

Cases: x next to the clustered roots of tests/nearroot.py (fp32 and bf16
neighbours, where fp64 and compensated Horner cannot fix the sign), random
polynomials of every degree the header accepts, random x next to real roots of
random polynomials, zero coefficients, x = +-0, subnormals, and exponents
spread far enough to leave the window.  Wherever the routine answers it must be
exact; it must answer for every input of the stated domain (|x| in
[2^-16, 2^16], coefficient magnitudes within a factor 2^40 of each other,
n <= 6); and it declines exactly when the terms' aligned bit span, computed
here from the definitions, exceeds the window.  Compensated Horner must match
the exact sign on every n <= 4 fixture (clustered roots, and exact roots of
cubics with a full 24-bit x), and is shown to miss some n = 6 ones.
"""
import math
import os
import shutil
import subprocess
import sys
from fractions import Fraction

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import nearroot  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gr_kan_rational_amd", "csrc")
WINDOW_BITS = 256

HARNESS = r"""
#include "grkan_qsign.h"
#include <cstdio>
template <int N> void run(const float *b, float x) {
    float bb[N];
    for (int j = 0; j < N; ++j) bb[j] = b[j];
    int s = 0;
    const bool ok = grkan::qsign_integer<N>(x, bb, s);
    printf("%d %d %d\n", ok ? 1 : 0, s, grkan::qsign_compensated<N>(x, bb));
}
int main() {
    int n;
    while (scanf("%d", &n) == 1) {
        float b[8], x;
        for (int j = 0; j < n; ++j)
            if (scanf("%a", &b[j]) != 1) return 2;
        if (scanf("%a", &x) != 1) return 2;
        switch (n) {
            case 1: run<1>(b, x); break;
            case 2: run<2>(b, x); break;
            case 3: run<3>(b, x); break;
            case 4: run<4>(b, x); break;
            case 5: run<5>(b, x); break;
            case 6: run<6>(b, x); break;
            case 7: run<7>(b, x); break;
            case 8: run<8>(b, x); break;
            default: return 3;
        }
    }
    return 0;
}
"""


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("qsign")
    src = d / "qsign_check.cpp"
    src.write_text(HARNESS)
    exe = d / "qsign_check"
    # -ffp-contract=off: g++ ignores the header's clang pragma that keeps the
    # error-free transformations from being fused into FMAs
    subprocess.run([gxx, "-O2", "-std=c++17", "-ffp-contract=off", "-Wall", "-Wno-unknown-pragmas", "-I", CSRC,
                    str(src), "-o", str(exe)], check=True)

    def run(cases):
        inp = "".join(f"{len(b)} " + " ".join(float(v).hex() for v in b) + f" {float(x).hex()}\n"
                      for b, x in cases)
        r = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr
        out = [tuple(map(int, line.split())) for line in r.stdout.splitlines()]  # ok, s, compensated
        assert len(out) == len(cases)
        return out

    return run


def exact_sign(b, x):
    X = Fraction(float(x))
    q = sum(Fraction(float(c)) * X ** j for j, c in enumerate(b))
    return (q > 0) - (q < 0)


def odd_split(v):
    """|v| = m 2^e with m odd (v a nonzero finite fp32 value)."""
    m, e = math.frexp(abs(float(v)))
    m, e = int(m * 2 ** 24), e - 24  # exact: fp32 has 24 significant bits
    while m % 2 == 0:
        m //= 2
        e += 1
    return m, e


def span_bits(b, x):
    """Top bit of the largest aligned term over the smallest quantum (x != 0), +3."""
    X, e = odd_split(x)
    terms = [(odd_split(c), j) for j, c in enumerate(b) if c != 0]
    if not terms:
        return 0
    g = [f + j * e for (_, f), j in terms]
    G = min(g)
    return max(B.bit_length() + gj - G + j * X.bit_length() for ((B, _), j), gj in zip(terms, g)) + 3


def check(harness, cases, expect_all_ok=False):
    out = harness(cases)
    n_ok = 0
    for (b, x), (ok, s, _) in zip(cases, out):
        if x != 0 and all(np.isfinite(b)) and np.isfinite(x):
            assert ok == (span_bits(b, x) <= WINDOW_BITS - 1), (list(map(float, b)), float(x))
        if ok:
            n_ok += 1
            assert s == exact_sign(b, x), (list(map(float, b)), float(x), s)
        elif expect_all_ok:
            raise AssertionError(f"declined inside the stated domain: {list(map(float, b))} {float(x)}")
    return n_ok


def test_clustered_roots_fp32_and_bf16(harness):
    cases = []
    for n, sets in nearroot.CLUSTERS.items():
        for roots in sets:
            b = nearroot.coefficients(roots)
            for r in sorted(set(roots)):
                for x in nearroot.neighbours(r, 60):
                    cases.append((b, x))
                for x in nearroot.neighbours(r, 20, "bf16"):
                    cases.append((b, x))
    assert check(harness, cases, expect_all_ok=True) == len(cases)
    # the fixtures do reach below fp64: some signs are decided by terms under 2^-100 of the sum of |terms|
    deep = 0
    for b, x in cases:
        X = Fraction(float(x))
        q = sum(Fraction(float(c)) * X ** j for j, c in enumerate(b))
        scale = sum(abs(Fraction(float(c))) * abs(X) ** j for j, c in enumerate(b))
        deep += q != 0 and abs(q) < scale / 2 ** 100
    assert deep > 0


def test_random_polynomials_in_domain(harness):
    rng = np.random.default_rng(11)
    cases = []
    for _ in range(6000):
        n = int(rng.integers(1, 7))
        b = (rng.choice([-1, 1], n) * np.exp2(rng.uniform(-20, 20, n))).astype(np.float32)
        if rng.random() < 0.2:
            b[rng.integers(0, n)] = 0
        x = np.float32(rng.choice([-1, 1]) * np.exp2(rng.uniform(-16, 16)))
        cases.append((b, x))
    assert check(harness, cases, expect_all_ok=True) == len(cases)


def test_near_real_roots_of_random_polynomials(harness):
    rng = np.random.default_rng(12)
    cases = []
    for _ in range(1500):
        n = int(rng.integers(2, 7))
        b = rng.standard_normal(n).astype(np.float32)
        for r in np.roots(b[::-1].astype(np.float64)):
            if abs(r.imag) < 1e-12 and 2.0 ** -16 < abs(r.real) < 2.0 ** 16:
                for x in nearroot.neighbours(np.float32(r.real), 3):
                    cases.append((b, x))
    assert check(harness, cases, expect_all_ok=True) == len(cases)


def test_degrees_up_to_eight_and_special_values(harness):
    rng = np.random.default_rng(13)
    f = np.float32
    cases = []
    for n in (7, 8):
        for _ in range(500):
            cases.append((rng.standard_normal(n).astype(np.float32), f(rng.standard_normal() * 2)))
    b = np.array([0.5, -1.25, 0, 2.0], np.float32)
    for x in (f(0), -f(0), f(1e-40), f(-1e-45), f(3e38), f(1e-30), f(1.0)):
        cases.append((b, x))
    cases.append((np.zeros(4, np.float32), f(1.5)))                  # b = 0: q = 0
    cases.append((np.array([0, 0, 1e-40, 0], np.float32), f(-2.0)))   # subnormal coefficient
    cases.append((np.array([-0.0, 0.0, 0.0], np.float32), f(0)))      # q(0) = -0
    check(harness, cases)
    out = harness(cases[-3:])
    assert [r[:2] for r in out] == [(1, 0), (1, 1), (1, 0)]


def test_window_is_left_only_for_wide_spans(harness):
    rng = np.random.default_rng(14)
    cases = []
    for _ in range(3000):
        n = int(rng.integers(2, 7))
        b = (rng.choice([-1, 1], n) * np.exp2(rng.uniform(-100, 100, n))).astype(np.float32)
        x = np.float32(rng.choice([-1, 1]) * np.exp2(rng.uniform(-100, 100)))
        cases.append((b, x))
    n_ok = check(harness, cases)
    assert 0 < n_ok < len(cases)  # both kinds occur; every answer given is exact


def test_non_finite_inputs_are_declined(harness):
    f = np.float32
    cases = [(np.array([1, 2], np.float32), f(np.inf)), (np.array([1, 2], np.float32), f(np.nan)),
             (np.array([np.inf, 2], np.float32), f(1)), (np.array([1, np.nan], np.float32), f(0))]
    assert [r[0] for r in harness(cases)] == [0, 0, 0, 0]


def cubic_exact_roots(count, seed):
    """q(y) = (2^k y - X)(2^(k+b-24) y^2 + 2^b y + 2^a), a = b + 24 - k: fp32 coefficients, and
    x = X / 2^k (a full 24-bit mantissa) an exact root; with its two fp32 neighbours."""
    rng = np.random.default_rng(seed)
    cases = []
    for t in range(count):
        X = int(rng.integers(2 ** 23, 2 ** 24)) | 1
        k = int(rng.integers(20, 26))
        b = int(rng.integers(-30, 0))
        sgn = 1 if t % 2 else -1
        f2 = [Fraction(2) ** (b + 24 - k), Fraction(2) ** b, sgn * Fraction(2) ** (k + b - 24)]
        p = [Fraction(0)] * 4
        for i, u in enumerate([-Fraction(X), Fraction(2) ** k]):
            for j, v in enumerate(f2):
                p[i + j] += u * v
        b32 = np.array([float(v) for v in p], np.float32)
        if not all(Fraction(float(v)) == w for v, w in zip(b32, p)):
            continue  # a coefficient needs more than 24 bits
        x = np.float32(X / 2 ** k)
        for xx in (x, np.nextafter(x, np.float32(0)), np.nextafter(x, np.float32(9))):
            cases.append((b32, xx))
    return cases


def test_compensated_horner_where_the_kernels_use_it(harness):
    cases = []
    for n in (4,):
        for roots in nearroot.CLUSTERS[n]:
            b = nearroot.coefficients(roots)
            for r in sorted(set(roots)):
                cases += [(b, x) for x in nearroot.neighbours(r, 60)]
                cases += [(b, x) for x in nearroot.neighbours(r, 20, "bf16")]
    cubic = cubic_exact_roots(1500, 15)
    assert len(cubic) > 1500
    cases += cubic
    rng = np.random.default_rng(16)
    for _ in range(1500):
        n = int(rng.integers(2, 5))
        b = rng.standard_normal(n).astype(np.float32)
        for r in np.roots(b[::-1].astype(np.float64)):
            if abs(r.imag) < 1e-12 and 2.0 ** -16 < abs(r.real) < 2.0 ** 16:
                cases += [(b, x) for x in nearroot.neighbours(np.float32(r.real), 3)]
    out = harness(cases)
    wrong = [(list(map(float, b)), float(x)) for (b, x), (_, _, c) in zip(cases, out) if c != exact_sign(b, x)]
    assert not wrong, wrong[:5]


def test_compensated_horner_misses_five_fold_roots(harness):
    """Why the kernels decide n >= 5 exactly: next to (x - 2.75)^5, compensated Horner in fp64
    returns 0 for some fp32 x whose q(x) is not 0."""
    b = nearroot.coefficients([2.75] * 5)
    cases = [(b, x) for x in nearroot.neighbours(2.75, 60)]
    out = harness(cases)
    wrong = sum(c != exact_sign(bb, x) for (bb, x), (_, _, c) in zip(cases, out))
    assert wrong > 0
    assert all(ok == 1 and s == exact_sign(bb, x) for (bb, x), (ok, s, _) in zip(cases, out))
