"""fp64 CPU oracle for a Chebyshev-KAN layer (forward and backward).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this module; it shares no
code with the HIP path.

What is computed.  "PolyKAN: Efficient Fused GPU Operators for Polynomial
Kolmogorov-Arnold Network Variants" (abstract page, arXiv 2511.14852) takes
the Chebyshev KAN as its case study but prints no formula.  Reading (the
common formulation of that layer): every input x_i is squashed into [-1, 1]
by t_i = tanh(x_i), expanded in Chebyshev polynomials of the first kind,
T_0 = 1, T_1 = t, T_{k+1} = 2 t T_k - T_{k-1}, and each output is a learned
combination of all of them:

    y[r, o] = sum_i sum_{k=0..D} C[o, i, k] T_k(t[r, i])

The coefficients are stored [d_out][d_in][D + 1] (degree fastest), so that
y = basis(x) C^T with basis(x)[r, i (D + 1) + k] = T_k(t[r, i]) -- a matrix
product over K = d_in (D + 1).  In the bf16 layer the contraction takes each
basis value rounded to bf16 (round to nearest, ties to even).

Backward, by the chain rule with dy = dL/dy (bf16):

    dC[o, i, k] = sum_r dy[r, o] T_k(t[r, i])          (dC = dy^T basis)
    dx[r, i]    = (1 - t^2) sum_k T_k'(t) G[r, i, k],   G = dy C   (fp64 here)

with T_k' = k U_{k-1} (U: Chebyshev polynomials of the second kind, U_0 = 1,
U_1 = 2t, U_{k+1} = 2 t U_k - U_{k-1}).

Where the rounding is not unique.  The GPU evaluates tanh and the recurrence
in fp32; where the exact basis value lies within that accuracy of a bf16
midpoint, both neighbours are correct operands.  ``basis_error`` bounds the
fp32 error (absolute; |t| <= 1 and |T_k| <= 1 on [-1, 1]): t within 2^-21
of tanh(x) moves T_k by at most |T_k'| 2^-21 <= k^2 2^-21, and the k
recurrence steps' roundings (2^-24 each, carried forward with gain at most
k + 1) add less than k^2 2^-23; (k^2 + 1) 2^-20 covers both.  Flagged
elements feed the ``*_amb`` allowances.

dx is compared elementwise against ``dxerr``, the first-order bound of the
same fp32 evaluation: the products of G accumulated in fp32 over K = d_out
terms (K 2^-24 of |dy||C|) and G then rounded to bf16 (half a bf16 unit), T_k'
evaluated at a t off by 2^-21 (at most max|T_k''| = k^2 (k^2 - 1) / 3 times
that) with its own recurrence roundings (k^2 2^-22), 1 - t^2 off by 2^-20,
and the final products and sum.
"""
from __future__ import annotations

import numpy as np

from . import layer
from . import oracle


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (the bf16 minimum normal spacing below it)."""
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.frexp(a)[1] - 8)


def basis_error(k: np.ndarray) -> np.ndarray:
    """Absolute fp32 error bound of the GPU's T_k (see the module docstring)."""
    k = np.asarray(k, dtype=np.float64)
    return (k * k + 1) * 2.0 ** -20


def chebyshev_t(t: np.ndarray, degree: int) -> np.ndarray:
    """T_0..T_degree at every t, by the three-term recurrence: shape t.shape + (degree + 1,)."""
    t = np.asarray(t, dtype=np.float64)
    out = np.empty(t.shape + (degree + 1,), dtype=np.float64)
    out[..., 0] = 1.0
    if degree >= 1:
        out[..., 1] = t
    for k in range(1, degree):
        out[..., k + 1] = 2.0 * t * out[..., k] - out[..., k - 1]
    return out


def chebyshev_dt(t: np.ndarray, degree: int) -> np.ndarray:
    """T_k'(t) = k U_{k-1}(t), k = 0..degree: shape t.shape + (degree + 1,)."""
    t = np.asarray(t, dtype=np.float64)
    u = np.empty(t.shape + (max(degree, 1),), dtype=np.float64)   # U_0 .. U_{degree-1}
    u[..., 0] = 1.0
    if degree >= 2:
        u[..., 1] = 2.0 * t
    for k in range(1, degree - 1):
        u[..., k + 1] = 2.0 * t * u[..., k] - u[..., k - 1]
    out = np.zeros(t.shape + (degree + 1,), dtype=np.float64)
    for k in range(1, degree + 1):
        out[..., k] = k * u[..., k - 1]
    return out


def basis_operand(x_bits: np.ndarray, degree: int):
    """(bf16 basis [rows, d_in (D+1)], ambiguity width, exact basis) for bf16 x [rows, d_in]."""
    x = oracle.to_f64(np.ascontiguousarray(x_bits), "bf16")
    t = np.tanh(x)
    T = chebyshev_t(t, degree)                                   # [rows, d_in, D+1]
    err = basis_error(np.arange(degree + 1))
    lo, hi = layer.bf16_round(T - err), layer.bf16_round(T + err)
    rows = x.shape[0]
    return (layer.bf16_round(T).reshape(rows, -1), np.where(lo != hi, hi - lo, 0.0).reshape(rows, -1),
            T.reshape(rows, -1))


def forward(x_bits: np.ndarray, C_bits: np.ndarray, degree: int) -> dict:
    """y [rows, d_out] = bf16(basis(x)) C^T in fp64, with ``amb`` (rounding ambiguity) and
    ``mag`` (sum of |products|) of the same shape; C is [d_out, d_in, D+1] bf16 bits."""
    rows, d_in = np.asarray(x_bits).shape
    C = layer.bf16_value(C_bits).reshape(-1, d_in * (degree + 1))
    bb, width, _ = basis_operand(x_bits, degree)
    ac = np.abs(C)
    return {"y": bb @ C.T, "amb": width @ ac.T, "mag": np.abs(bb) @ ac.T}


def backward(x_bits: np.ndarray, dy_bits: np.ndarray, C_bits: np.ndarray, degree: int) -> dict:
    """dC [d_out, d_in, D+1] with its terms' L2 norms ``dC_norm`` and allowance ``dC_amb``;
    dx [rows, d_in] with its error bound ``dxerr`` (see the module docstring)."""
    x_bits = np.asarray(x_bits)
    rows, d_in = x_bits.shape
    nb = degree + 1
    dy = layer.bf16_value(dy_bits).reshape(rows, -1)
    d_out = dy.shape[1]
    C = layer.bf16_value(C_bits).reshape(d_out, d_in * nb)
    bb, width, _ = basis_operand(x_bits, degree)
    out = {"dC": (dy.T @ bb).reshape(d_out, d_in, nb),
           "dC_amb": (np.abs(dy).T @ width).reshape(d_out, d_in, nb),
           "dC_norm": np.sqrt((dy * dy).T @ (bb * bb)).reshape(d_out, d_in, nb)}
    x = oracle.to_f64(x_bits, "bf16")
    t = np.tanh(x)
    dT = chebyshev_dt(t, degree)                                 # [rows, d_in, D+1]
    G = (dy @ C).reshape(rows, d_in, nb)
    Gmag = (np.abs(dy) @ np.abs(C)).reshape(rows, d_in, nb)
    s = 1.0 - t * t
    out["dx"] = s * np.sum(dT * G, axis=-1)
    k = np.arange(nb, dtype=np.float64)
    m2 = k * k * (k * k - 1) / 3.0                             # max |T_k''| on [-1, 1]
    adT = np.abs(dT)
    acc = d_out * 2.0 ** -24 * Gmag
    per_k = adT * (acc + 0.5 * bf16_ulp(np.abs(G) + acc)) + (m2 * 2.0 ** -21 + k * k * 2.0 ** -22) * Gmag
    out["dxerr"] = s * np.sum(per_k, axis=-1) + (2.0 ** -20 + 16 * 2.0 ** -24) * np.sum(adT * Gmag, axis=-1)
    return out
