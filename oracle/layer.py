"""fp64 CPU oracle for the GR-KAN layer's forward: z = F(x) W^T.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this module; it shares no
code with the HIP path.

What is computed.  A GR-KAN layer applies the group-rational activation F to
its d_in inputs and maps the result linearly to d_out outputs ("FlashKAT:
Understanding and Addressing Performance Bottlenecks in the Kolmogorov-Arnold
Transformer", Paper-Notes page, section "1. 性能瓶颈诊断", Insight 2: the
rational's (2m + 2n + 3) d_in FLOPs against the linear map's 2 d_in d_out).
The page prints no bias, so none is added.  In the bf16 layer the contraction
takes F's value rounded to bf16 (round to nearest, ties to even), as a bf16
matrix unit consumes it:

    z[r, o] = sum_c bf16(F_g(c)(x[r, c])) * W[o, c]

F comes from ``oracle.run`` (fp64, pinned by its own tests); the rounding is
written out here; the sum is a plain fp64 matrix product.

Where the rounding is not unique.  F itself is only known to the GPU to fp32
accuracy; where the exact F lies within that accuracy of a point halfway
between two bf16 values, both neighbours are correct roundings.  Such
elements are flagged, and ``amb`` bounds what choosing the other neighbour
can change in z.  ``mag`` = sum |bf16(F)| |W| scales the fp32 accumulation
error.

Backward.  With dz = dL/dz (bf16), the chain rule through z = bf16(F) W^T
gives the weight gradient dW = dz^T bf16(F(x)) and dL/dF = dz W.  The GPU
rounds dz W (accumulated in fp32) to bf16 before the activation's backward,
as a bf16 layer does; the oracle does the same from the fp64 product and
flags the elements whose fp64 product lies within fp32 accumulation error
(d_out 2^-24 sum |dz||W|) of a bf16 rounding boundary.  dx, dA, dB are then
the activation oracle's backward at dy = bf16(dz W); for the flagged elements
``dx_amb``, ``dA_amb``, ``dB_amb`` bound what the other admissible rounding
changes (dx and the terms are linear in dy).
"""
from __future__ import annotations

import numpy as np

from . import oracle

# fp32 evaluation error of F, relative to its first-order rounding scale
# (oracle field "ymag"): generous against the few roundings of a Horner
# evaluation and a reciprocal.
F32_ERROR = 16.0 * 2.0 ** -24


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Nearest bf16 value of each fp64 value, ties to even (8 significant bits;
    the bf16 exponent range is fp32's, subnormals down to 2^-133)."""
    v = np.asarray(v, dtype=np.float64)
    mant, exp = np.frexp(v)                 # v = mant * 2**exp, 0.5 <= |mant| < 1
    shift = np.maximum(exp - 8, -133)       # exponent of one unit in the last place
    q = np.rint(np.ldexp(v, -shift))        # round half to even
    return np.ldexp(q, shift)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """fp64 value of bf16 bit patterns (uint16)."""
    return oracle.to_f64(np.ascontiguousarray(bits, dtype=np.uint16), "bf16")


def activation_operand(x_bits: np.ndarray, A, B, n_groups: int):
    """(bf16(F(x)), ambiguity width) for x given as bf16 bits [rows, d_in]: the width is
    one bf16 step where the rounding is not unique (see the module docstring), else 0."""
    res = oracle.run(x_bits, A, B, n_groups, io="bf16")
    f, fmag = res["y"], res["ymag"]
    err = F32_ERROR * fmag
    fb = bf16_round(f)
    lo, hi = bf16_round(f - err), bf16_round(f + err)
    width = np.where(lo != hi, hi - lo, 0.0)
    return fb, width


def forward(x_bits: np.ndarray, A, B, W_bits: np.ndarray, n_groups: int) -> dict:
    """z [rows, d_out] = bf16(F(x)) W^T in fp64, with ``amb`` and ``mag`` (same shape) and
    ``n_ambiguous`` (flagged elements of bf16(F(x)))."""
    x_bits = np.asarray(x_bits)
    rows, d_in = x_bits.shape
    W = bf16_value(W_bits).reshape(-1, d_in)
    fb, width = activation_operand(x_bits, A, B, n_groups)
    aw = np.abs(W)
    return {"z": fb @ W.T, "amb": width @ aw.T, "mag": np.abs(fb) @ aw.T,
            "n_ambiguous": int(np.count_nonzero(width))}


def bf16_bits(values: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of values that are exactly representable in bf16."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    f = v.astype(np.float32)
    if not np.array_equal(f.astype(np.float64), v):
        raise ValueError("not bf16 values")
    b = f.view(np.uint32)
    if np.any(b & 0xFFFF):
        raise ValueError("not bf16 values")
    return (b >> 16).astype(np.uint16)


def upstream(dz_bits: np.ndarray, W_bits: np.ndarray):
    """(bf16(dz W), ambiguity width) for bf16 dz [rows, d_out], W [d_out, d_in]."""
    dz = bf16_value(dz_bits)
    W = bf16_value(W_bits)
    k = W.shape[0]
    dy = dz @ W
    err = k * 2.0 ** -24 * (np.abs(dz) @ np.abs(W))
    lo, hi = bf16_round(dy - err), bf16_round(dy + err)
    return bf16_round(dy), np.where(lo != hi, hi - lo, 0.0)


def backward(x_bits: np.ndarray, dz_bits: np.ndarray, A, B, W_bits: np.ndarray, n_groups: int) -> dict:
    """Layer backward: dW [d_out, d_in] with its terms' L2 norms ``dW_norm`` and allowance
    ``dW_amb``; dx [rows, d_in] with ``dxmag`` and ``dx_amb``; dA, dB with the activation
    oracle's norms (nA, nB, mA, mB) and allowances ``dA_amb``, ``dB_amb``."""
    x_bits = np.asarray(x_bits)
    rows, d_in = x_bits.shape
    dz = bf16_value(dz_bits).reshape(rows, -1)
    fb, wf = activation_operand(x_bits, A, B, n_groups)
    out = {"dW": dz.T @ fb, "dW_amb": np.abs(dz).T @ wf, "dW_norm": np.sqrt((dz * dz).T @ (fb * fb))}
    dyb, wy = upstream(dz_bits, W_bits)
    act = oracle.run(x_bits, A, B, n_groups, dy=bf16_bits(dyb), io="bf16")
    for k in ("dx", "dxmag", "dA", "dB", "nA", "nB", "mA", "mB"):
        out[k] = act[k]
    out["dx_amb"] = np.zeros_like(act["dx"])
    out["dA_amb"] = np.zeros_like(act["dA"])
    out["dB_amb"] = np.zeros_like(act["dB"])
    flagged = np.flatnonzero(wy.ravel())
    out["n_ambiguous_dy"] = int(flagged.size)
    if flagged.size:
        ones = np.full(flagged.size, 0x3F80, dtype=np.uint16)   # dy = 1: the derivatives in dy
        dyone = np.zeros(rows * d_in, dtype=np.uint16)
        dyone[flagged] = ones
        rec = oracle.points(x_bits, A, B, n_groups, flagged, dy=dyone.reshape(rows, d_in), io="bf16")
        w = wy.ravel()[flagged]
        out["dx_amb"].ravel()[flagged] = w * np.abs(rec[:, oracle.DX])
        g = (flagged % d_in) // (d_in // n_groups)
        na = out["dA"].shape[1]
        for i in range(na):
            np.add.at(out["dA_amb"][:, i], g, w * np.abs(rec[:, oracle.TA + i]))
        for j in range(out["dB"].shape[1]):
            np.add.at(out["dB_amb"][:, j], g, w * np.abs(rec[:, oracle.TB + j]))
    return out
