"""Pins of the Chebyshev-KAN oracle (oracle/chebykan.py) to things other than
itself: numpy's Chebyshev-series routines and the closed form T_k(cos θ) =
cos(kθ), brute-force sums, central finite differences of the loss for dx, the
linearity of the loss in C for dC, and an fp32 evaluation against the basis
error bound.
"""
import math

import numpy as np
from numpy.polynomial import chebyshev as npcheb

from gr_kan_rational_amd import synth
from oracle import chebykan as ck
from oracle import layer
from oracle import oracle as orc

D = 7


def test_basis_matches_numpy_and_the_closed_form():
    t = np.linspace(-1, 1, 1001)
    T = ck.chebyshev_t(t, D)
    dT = ck.chebyshev_dt(t, D)
    for k in range(D + 1):
        e = np.zeros(k + 1)
        e[k] = 1
        assert np.allclose(T[:, k], npcheb.chebval(t, e), atol=1e-13)
        assert np.allclose(T[:, k], np.cos(k * np.arccos(t)), atol=1e-12)
        assert np.allclose(dT[:, k], npcheb.chebval(t, npcheb.chebder(e)), atol=1e-11)


def inputs(rows=3, d_in=8, d_out=4, seed=41):
    w = synth.custom("cheby-pin", rows, d_in, 1, io="bf16", seed=seed, d_out=d_out, cheby=D)
    return synth.make_inputs(w)


def exact_basis(xv):
    """T_k(tanh x) by cos(k arccos t), k = 0..D: [..., D + 1]."""
    th = np.arccos(np.tanh(xv))
    return np.cos(np.arange(D + 1) * th[..., None])


def test_forward_brute_force():
    inp = inputs()
    x, C = inp["x"], inp["W"]
    res = ck.forward(x, C, D)
    xv, cv = orc.to_f64(x, "bf16"), orc.to_f64(C.reshape(C.shape[0], -1), "bf16").reshape(C.shape)
    Tb = layer.bf16_round(exact_basis(xv))
    rows, d_in = x.shape
    for r in range(rows):
        for o in range(C.shape[0]):
            ref = math.fsum(cv[o, i, k] * Tb[r, i, k] for i in range(d_in) for k in range(D + 1))
            assert abs(res["y"][r, o] - ref) <= 1e-12 * (abs(ref) + 1e-12)


def test_backward_dC_brute_force_and_linearity():
    inp = inputs(rows=5, d_in=8, d_out=3, seed=42)
    x, C, dy = inp["x"], inp["W"], inp["dz"]
    res = ck.backward(x, dy, C, D)
    xv, dyv = orc.to_f64(x, "bf16"), orc.to_f64(dy, "bf16")
    Tb = layer.bf16_round(exact_basis(xv))
    for o in range(3):
        for i in range(8):
            for k in range(D + 1):
                ref = math.fsum(dyv[r, o] * Tb[r, i, k] for r in range(5))
                assert abs(res["dC"][o, i, k] - ref) <= 1e-12 * (abs(ref) + 1e-12)
    # the loss sum dy * y is linear in C: doubling C[o, i, k] adds C[o, i, k] dC[o, i, k]
    cv = orc.to_f64(C.reshape(3, -1), "bf16").reshape(C.shape)
    base = math.fsum((dyv * ck.forward(x, C, D)["y"]).ravel())
    for o, i, k in [(0, 0, 0), (2, 5, 7), (1, 3, 2)]:
        C2 = C.copy()
        C2[o, i, k] = synth.bf16_bits(np.float32([2 * cv[o, i, k]]))[0]
        dl = math.fsum((dyv * ck.forward(x, C2, D)["y"]).ravel()) - base
        assert abs(dl - cv[o, i, k] * res["dC"][o, i, k]) <= 1e-10 * (abs(dl) + 1e-12)


def test_backward_dx_finite_differences():
    # dx is the derivative of L(x) = sum dy * y(x) with the exact (unrounded) basis
    inp = inputs(rows=2, d_in=8, d_out=5, seed=43)
    x, C, dy = inp["x"], inp["W"], inp["dz"]
    res = ck.backward(x, dy, C, D)
    xv, dyv = orc.to_f64(x, "bf16"), orc.to_f64(dy, "bf16")
    cv = orc.to_f64(C.reshape(5, -1), "bf16").reshape(C.shape)

    def loss(xm):
        return float(np.einsum("ro,oik,rik->", dyv, cv, exact_basis(xm)))

    for r in range(2):
        for i in range(8):
            h = 1e-6
            xp, xm = xv.copy(), xv.copy()
            xp[r, i] += h
            xm[r, i] -= h
            fd = (loss(xp) - loss(xm)) / (2 * h)
            assert abs(fd - res["dx"][r, i]) <= 1e-6 * (abs(res["dx"][r, i]) + 1e-3)


def test_basis_error_bound_covers_an_fp32_evaluation():
    rng = np.random.default_rng(5)
    x32 = (rng.standard_normal(200000) * 2).astype(np.float32)
    t32 = np.tanh(x32)                                   # float32 tanh
    T32 = np.empty((x32.size, D + 1), np.float32)
    T32[:, 0] = 1
    T32[:, 1] = t32
    for k in range(1, D):
        T32[:, k + 1] = np.float32(2) * t32 * T32[:, k] - T32[:, k - 1]
    exact = ck.chebyshev_t(np.tanh(x32.astype(np.float64)), D)
    assert np.all(np.abs(T32 - exact) <= ck.basis_error(np.arange(D + 1)))
