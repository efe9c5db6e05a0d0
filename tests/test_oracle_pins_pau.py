"""Pins of the fp64 oracle at other degrees (m, n) and group counts: the PAU family.

The pages state that the kernel restructuring carries over to PAU and its
variants ([FlashKAT notes], section "局限性与未来工作"); PAU is P/(1 + |Q|)
with free numerator degree m and denominator degree n (Q without constant
term).  GR-KAN is m = 5, n = 4 with 8 groups; n = 0 is a plain polynomial.
Each test pins the oracle to a fact from outside it: numpy's polynomial
routines, sympy's symbolic derivatives, exact rational arithmetic (Python
fractions), finite differences and brute-force sums.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as orc

rng = np.random.default_rng(4321)
PV = np.polynomial.polynomial
XS = np.array([-3.5, -1.25, -0.3, -1e-3, 0.0, 2e-3, 0.5, 0.875, 1.0, 2.75, 4.0], dtype=np.float32)
PAIRS = [(2, 1), (3, 2), (4, 3), (6, 5), (7, 6), (4, 4), (5, 0), (0, 3)]


def coefs(m, n, n_g=1, scale=0.5):
    A = (rng.standard_normal((n_g, m + 1)) * scale).astype(np.float32)
    B = (rng.standard_normal((n_g, n)) * scale).astype(np.float32)
    return A, B


def recs(xs, a, b, m, n, dy=1.0):
    return np.array([orc.point(float(x), dy, a, b, m, n) for x in xs])


@pytest.mark.parametrize("m", range(0, 8))
@pytest.mark.parametrize("n", [0, 1, 3, 6])
def test_polynomial_when_denominator_vanishes(m, n):
    """b = 0 => F = P (numpy polyval), dF/dx = P' (polyder), dF/da_i = x^i, dF/db_j = 0."""
    a = (rng.standard_normal(m + 1) * 0.7).astype(np.float32).astype(np.float64)
    ta, tb, nout = orc.layout(m, n)
    r = recs(XS, a, np.zeros(n), m, n, dy=1.5)
    assert r.shape == (XS.size, nout)
    x = XS.astype(np.float64)
    np.testing.assert_allclose(r[:, orc.F], PV.polyval(x, a), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(r[:, orc.DX], 1.5 * PV.polyval(x, PV.polyder(a)), rtol=1e-14, atol=1e-14)
    for i in range(m + 1):
        np.testing.assert_allclose(r[:, ta + i], 1.5 * x ** i, rtol=1e-15, atol=0)
    assert np.all(r[:, tb:tb + n] == 0) and np.all(r[:, orc.SIGN] == 0) and np.all(r[:, orc.DEN] == 1)


@pytest.mark.parametrize("m,n", [(3, 2), (7, 6), (2, 1), (6, 5), (4, 4)])
def test_monomial_denominator(m, n):
    """b = beta e_j (only b_j nonzero) => Q = beta x^j: F = P / (1 + |beta| |x|^j) with P from numpy,
    sign(Q) = sign(beta x^j), D = 1 + |beta x^j|, dF/da_i = x^i / D.  Pins which b multiplies which
    power and the layout of the record."""
    a = (rng.standard_normal(m + 1) * 0.7).astype(np.float32).astype(np.float64)
    x = XS.astype(np.float64)
    ta, tb, _ = orc.layout(m, n)
    for j in range(1, n + 1):
        beta = float(np.float32(rng.uniform(0.2, 1.5) * rng.choice([-1, 1])))
        b = np.zeros(n)
        b[j - 1] = beta
        r = recs(XS, a, b, m, n)
        D = 1 + np.abs(beta * x ** j)
        np.testing.assert_allclose(r[:, orc.F], PV.polyval(x, a) / D, rtol=1e-14, atol=1e-15)
        np.testing.assert_array_equal(r[:, orc.SIGN], np.sign(beta * x ** j))
        np.testing.assert_allclose(r[:, orc.DEN], D, rtol=1e-15)
        for i in range(m + 1):
            np.testing.assert_allclose(r[:, ta + i], x ** i / D, rtol=1e-14, atol=0)


@pytest.mark.parametrize("m,n", PAIRS)
def test_derivatives_match_sympy(m, n):
    """dF/dx, dF/da_i, dF/db_j against sympy's symbolic derivatives of P/(1+|Q|) at degrees (m, n),
    evaluated exactly at fp32 points."""
    import sympy as sp

    X = sp.Symbol("x", real=True)
    asym = sp.symbols(f"a0:{m + 1}", real=True)
    bsym = sp.symbols(f"b1:{n + 1}", real=True) if n else ()
    P = sum(asym[i] * X ** i for i in range(m + 1))
    Q = sum(bsym[j - 1] * X ** j for j in range(1, n + 1)) if n else sp.Integer(0)
    Fs = P / (1 + sp.Abs(Q))
    dFx = sp.diff(Fs, X)
    dFa = [sp.diff(Fs, asym[i]) for i in range(m + 1)]
    dFb = [sp.diff(Fs, bsym[j]) for j in range(n)]
    ta, tb, _ = orc.layout(m, n)
    for trial in range(3):
        A, B = coefs(m, n)
        subs = {asym[i]: sp.Rational(float(A[0, i])) for i in range(m + 1)}
        subs.update({bsym[j]: sp.Rational(float(B[0, j])) for j in range(n)})
        for xv in (np.float32(-1.7), np.float32(-0.4), np.float32(0.9), np.float32(2.3)):
            s2 = dict(subs)
            s2[X] = sp.Rational(float(xv))
            r = orc.point(float(xv), 1.0, A[0], B[0], m, n)
            assert r[orc.F] == pytest.approx(float(sp.N(Fs.subs(s2), 40)), rel=1e-13, abs=1e-14)
            assert r[orc.DX] == pytest.approx(float(sp.N(dFx.subs(s2), 40)), rel=1e-11, abs=1e-13)
            for i in range(m + 1):
                assert r[ta + i] == pytest.approx(float(sp.N(dFa[i].subs(s2), 40)), rel=1e-13, abs=1e-300)
            for j in range(n):
                assert r[tb + j] == pytest.approx(float(sp.N(dFb[j].subs(s2), 40)), rel=1e-11, abs=1e-13)


def _loss(x, dy, A, B, n_g, m, n):
    y = orc.run(x, A, B, n_g, m=m, n=n)["y"]
    return math.fsum((dy.astype(np.float64) * y).ravel())


@pytest.mark.parametrize("m,n", [(3, 2), (7, 6), (5, 0)])
def test_finite_differences(m, n):
    """dX by central differences of F; dA by exact differences (F is linear in a); dB by central
    differences in b_j, at degrees (m, n) over a [24, 16] tensor in 4 groups."""
    n_g, rows, d = 4, 24, 16
    x = rng.standard_normal((rows, d)).astype(np.float32)
    dy = rng.standard_normal((rows, d)).astype(np.float32)
    A, B = coefs(m, n, n_g, scale=0.4)
    r = orc.run(x, A, B, n_g, dy=dy, m=m, n=n)
    assert r["dA"].shape == (n_g, m + 1) and r["dB"].shape == (n_g, n)
    checked = 0
    for idx in range(0, x.size, 3):
        g = (idx % d) // (d // n_g)
        xv = float(x.ravel()[idx])
        h = 2.0 ** -20 * max(1.0, abs(xv))
        lo = orc.point(xv - h, 0.0, A[g], B[g], m, n)
        hi = orc.point(xv + h, 0.0, A[g], B[g], m, n)
        if lo[orc.SIGN] != hi[orc.SIGN]:
            continue
        fd = (hi[orc.F] - lo[orc.F]) / (2 * h) * float(dy.ravel()[idx])
        assert r["dx"].ravel()[idx] == pytest.approx(fd, rel=1e-6, abs=1e-8)
        checked += 1
    assert checked >= 0.9 * (x.size // 3)
    L0 = _loss(x, dy, A, B, n_g, m, n)
    for g in (0, 3):
        for i in range(m + 1):
            A2 = A.astype(np.float64).copy()
            A2[g, i] += 1.0
            diff = _loss(x, dy, A2, B, n_g, m, n) - L0
            assert diff == pytest.approx(r["dA"][g, i], rel=1e-8, abs=1e-9 * max(1.0, abs(L0)))
    hb = 1e-6
    idx = np.arange(x.size)
    for g in (1, 2):
        gi = idx[(idx % d) // (d // n_g) == g]
        for j in range(n):
            Bp = B.astype(np.float64).copy()
            Bm = Bp.copy()
            Bp[g, j] += hb
            Bm[g, j] -= hb
            if not np.array_equal(orc.points(x, A, Bp, n_g, gi, m=m, n=n)[:, orc.SIGN],
                                  orc.points(x, A, Bm, n_g, gi, m=m, n=n)[:, orc.SIGN]):
                continue  # a sign flip inside the step breaks the difference
            fd = (_loss(x, dy, A, Bp, n_g, m, n) - _loss(x, dy, A, Bm, n_g, m, n)) / (2 * hb)
            scale = r["nB"][g, j] * math.sqrt(x.size)
            assert fd == pytest.approx(r["dB"][g, j], rel=1e-5, abs=1e-6 * scale)


@pytest.mark.parametrize("m,n,n_g", [(3, 2, 4), (6, 5, 1), (5, 4, 16), (2, 1, 16)])
def test_group_sums_brute_force(m, n, n_g):
    """Group sums equal an fsum over per-element records taken one by one, for n_g = 1 (one
    shared function), n_g = d (one function per channel) and in between."""
    rows, d = 9, 16
    x = rng.standard_normal((rows, d)).astype(np.float32)
    dy = rng.standard_normal((rows, d)).astype(np.float32)
    A, B = coefs(m, n, n_g)
    rec = orc.points(x, A, B, n_g, np.arange(x.size), dy=dy, m=m, n=n)
    groups = (np.arange(x.size) % d) // (d // n_g)
    r = orc.run(x, A, B, n_g, dy=dy, m=m, n=n, nthreads=2)
    ta, _, _ = orc.layout(m, n)
    for g in range(n_g):
        for k in range(m + 1 + n):
            ref = math.fsum(rec[groups == g, ta + k])
            got = r["dA"][g, k] if k <= m else r["dB"][g, k - m - 1]
            assert got == pytest.approx(ref, rel=1e-13, abs=1e-15)


@pytest.mark.parametrize("n_g", [1, 4, 12])
def test_group_map_any_group_count(n_g):
    """Channel c uses group floor(c / d_g) for n_g = 1, n_g = d (per channel) and in between:
    group g gets a_0 = g + 1 and b = 0, so F == g + 1 on exactly its channels."""
    d, rows, m, n = 12, 3, 2, 1
    A = np.zeros((n_g, m + 1), np.float32)
    A[:, 0] = np.arange(1, n_g + 1)
    B = np.zeros((n_g, n), np.float32)
    x = rng.standard_normal((rows, d)).astype(np.float32)
    y = orc.run(x, A, B, n_g, m=m, n=n)["y"]
    expect = np.repeat(np.arange(1, n_g + 1), d // n_g)[None, :].repeat(rows, 0)
    assert np.array_equal(y, expect.astype(np.float64))


def _exact_sign(x, b):
    """sign of sum_j b_j x^j in exact rational arithmetic."""
    xf = Fraction(float(x))
    q = sum(Fraction(float(bj)) * xf ** (j + 1) for j, bj in enumerate(b))
    return (q > 0) - (q < 0)


@pytest.mark.parametrize("n", range(1, 8))
def test_sign_exact_near_roots(n):
    """At the fp32 neighbours of every real root of random degree-n denominators, the oracle's
    sign of Q equals the sign computed in exact rational arithmetic."""
    m = 1
    for trial in range(6):
        b = (rng.standard_normal(n) * 0.8).astype(np.float32)
        roots = PV.polyroots(b.astype(np.float64)) if n > 1 else np.array([])
        xs = [np.float32(0.0)]
        for rt in roots:
            if abs(rt.imag) > 1e-9 or not np.isfinite(rt.real) or abs(rt.real) > 1e6:
                continue
            c = np.float32(rt.real)
            for k in range(-3, 4):
                v = c
                step = np.float32(np.inf) if k > 0 else np.float32(-np.inf)
                for _ in range(abs(k)):
                    v = np.nextafter(v, step)
                xs.append(v)
        for xv in xs:
            s = orc.point(float(xv), 1.0, [0.0, 1.0], b, m, n)[orc.SIGN]
            assert s == _exact_sign(xv, b), (n, float(xv), b.tolist())


@pytest.mark.parametrize("k", [3, 5, 7])
def test_sign_beyond_quad_precision(k):
    """Q = x (x - 1)^k: at x = 1 + 2^-23 (and 1 - 2^-24) its value is 2^-23k (resp. -2^-24k) while
    its terms are of order binom(k, k/2): for k = 5, 7 the relative size is below even binary128's
    2^-113.  The oracle must return the exact sign: + above 1, -/+ below (odd k: -), 0 at 1."""
    coeffs = [math.comb(k, i) * (-1) ** (k - i) for i in range(k + 1)]  # (x - 1)^k, ascending
    b = np.array(coeffs, dtype=np.float32)  # b_j multiplies x^j, so Q = x (x - 1)^k
    n = k + 1
    above = float(np.nextafter(np.float32(1), np.float32(2)))
    below = float(np.nextafter(np.float32(1), np.float32(0)))
    assert orc.point(above, 1.0, [0.0, 1.0], b, 1, n)[orc.SIGN] == 1
    assert orc.point(below, 1.0, [0.0, 1.0], b, 1, n)[orc.SIGN] == -1
    assert orc.point(1.0, 1.0, [0.0, 1.0], b, 1, n)[orc.SIGN] == 0
    assert _exact_sign(np.float32(above), b) == 1 and _exact_sign(np.float32(below), b) == -1


def test_degree_limits():
    with pytest.raises(ValueError):
        orc.point(0.5, 1.0, np.zeros(17), [0.1], 16, 1)
    with pytest.raises(ValueError):
        orc.point(0.5, 1.0, [1.0], [], 0, -1)
    r = orc.point(0.5, 2.0, [3.0], [], 0, 0)  # constant: F = a_0, dX = 0, one term dY / 1
    assert r[orc.F] == 3.0 and r[orc.DX] == 0.0 and r[orc.T] == 2.0 and r.size == orc.layout(0, 0)[2]


@pytest.mark.parametrize("m,n", [(5, 4), (7, 6), (3, 2)])
def test_term_rounding_scales(m, n):
    """The per-term rounding scales dominate |term| and bound a plain numpy float32 evaluation of
    each term (Horner P and q, Q = x q, D = 1 + |Q|, t_a = dY x^i / D, t_b = -s dY P x^j / D^2)
    within 16 * 2^-24 of them, including points next to a root of Q where the fp32 Q has
    cancelled to a few ulps of its terms."""
    ta, tb, _ = orc.layout(m, n)
    nk = m + 1 + n
    u = 2.0 ** -24
    f = np.float32
    for trial in range(300):
        A, B = coefs(m, n, scale=0.6)
        a, b = A[0], B[0]
        if trial % 3 == 0 and n > 1:  # a point next to a real root of Q / x
            roots = [rt.real for rt in PV.polyroots(b.astype(np.float64)) if abs(rt.imag) < 1e-9]
            if not roots:
                continue
            xv = np.nextafter(f(roots[0]), f(np.inf))
        else:
            xv = f(rng.standard_normal() * 1.5)
        dyv = f(rng.standard_normal())
        r = orc.point(float(xv), float(dyv), a, b, m, n)
        terms, mags = r[ta:ta + nk], r[ta + nk:ta + 2 * nk]
        assert np.all(mags >= np.abs(terms) * (1 - 1e-15))
        P = f(0)
        for i in range(m, -1, -1):
            P = P * xv + a[i]
        q = f(0)
        for j in range(n - 1, -1, -1):
            q = q * xv + b[j]
        Q = q * xv
        D = f(1) + np.abs(Q)
        s = r[orc.SIGN]
        for i in range(m + 1):
            t32 = dyv * xv ** i / D
            assert abs(float(t32) - terms[i]) <= 16 * u * mags[i], (m, n, i, float(xv))
        for j in range(1, n + 1):
            t32 = -f(s) * dyv * P * xv ** j / (D * D)
            assert abs(float(t32) - terms[m + j]) <= 16 * u * mags[m + j], (m, n, j, float(xv))
