"""Seeded synthetic inputs for the GR-KAN activation: the one module that both
the HIP path's tests/benchmark and the fp64 oracle draw their inputs from.

It holds no part of the activation's arithmetic: it only draws normal
variates, scales them and (for bf16 I/O) rounds them to bf16.

Workloads.  The pages measure KAT models (ViT-style transformers with 197
tokens per image, batch 1024) whose MLPs are GR-KAN layers; the activation
tensors such a model feeds the GR-KAN kernels are [B, N, d].  These
generators stand in for them with i.i.d. normal data of the same shapes:

    tiny            [2, 8, 32]        fp32  dY ~ N(0, 1)     seed 1
    kat-t           [128, 197, 192]   fp32  dY ~ N(0, 1e-2)  seed 2
    kat-s-hid       [1024, 197, 1536] fp32  dY ~ N(0, 1e-2)  seed 3, group 0 numerator = identity
    kat-b           [1024, 197, 768]  fp32  dY ~ N(0, 1e-2)  seed 4
    kat-b-hid-bf16  [1024, 197, 3072] bf16  dY ~ N(0, 1e-2)  seed 5

with n_g = 8 groups, coefficients A [8, 6] and B [8, 4] ~ N(0, 0.5) and
X ~ N(0, 1) everywhere; N(0, s) means standard deviation s.

The PAU family (other numerator / denominator degrees m, n and group counts)
uses the same recipe with A [n_g, m+1] and B [n_g, n]:

    kat-b-pau       [1024, 197, 768]  fp32  n_g = 1,   (m, n) = (5, 4)  seed 6
    kat-b-r32       [1024, 197, 768]  fp32  n_g = 8,   (m, n) = (3, 2)  seed 7
    kat-b-r76       [1024, 197, 768]  fp32  n_g = 8,   (m, n) = (7, 6)  seed 8
    kat-b-poly5     [1024, 197, 768]  fp32  n_g = 8,   (m, n) = (5, 0)  seed 9
    kat-b-perchan   [1024, 197, 768]  fp32  n_g = 768, (m, n) = (5, 4)  seed 10 (one PAU per channel)

A GR-KAN layer (the activation followed by its linear map, bf16) adds the
weight W [d_out, d] ~ N(0, 1/sqrt(d)) (a fan-in scaled normal; the pages give
no initialisation for it), rounded to bf16:

    kat-b-layer1-bf16  X [1024, 197, 768]  -> 3072 outputs, n_g = 8  seed 11
    kat-b-layer2-bf16  X [1024, 197, 3072] -> 768 outputs,  n_g = 8  seed 12

(the two GR-KAN layers of a KAT-B MLP block).  Their backward takes the
upstream gradient dZ [rows, d_out] ~ N(0, 1e-2) (tensor 3 below) in place of
dY.

A Chebyshev-KAN layer (degree 7: 8 basis functions per input) draws its
coefficients C [d_out, d, 8] ~ N(0, 1/sqrt(8 d)) the same way, rounded to
bf16, and its upstream gradient as a layer's dZ:

    kat-b-cheby-bf16   X [1024, 197, 768]  -> 768 outputs             seed 13

(the shape of a KAT-B token mixer's input stands in for PolyKAN's speech,
audio and tabular workloads, which the pages do not size).

Recipe (reproducible, independent of the number of threads):
  * A then B (then W, for a layer) from ``numpy.random.default_rng(seed)``
    as float32 standard normals, multiplied by the std in float32;
  * X and dY in fixed chunks of 2**22 elements of the row-major tensor;
    chunk k of tensor t (t = 1 for X, 2 for dY, 3 for a layer's dZ) comes from
    ``PCG64(SeedSequence(seed, spawn_key=(t, k)))`` as float32 standard
    normals times the std in float32;
  * bf16 tensors are those float32 draws rounded to nearest-even bf16 and
    stored as uint16 bit patterns.
A run with fewer rows draws an exact prefix of the full tensors.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

CHUNK = 1 << 22


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq: int
    d: int
    n_groups: int
    io: str            # "f32" or "bf16" (I/O dtype of X, Y, dY, dX)
    coef_std: float
    x_std: float
    dy_std: float
    seed: int
    identity_group0: bool = False
    m: int = 5         # numerator degree (a_0..a_m)
    n: int = 4         # denominator degree (b_1..b_n)
    d_out: int = 0     # outputs of the layer's linear map (0: the activation alone)
    cheby: int = 0     # Chebyshev-KAN degree (0: a GR-KAN workload)

    @property
    def rows(self) -> int:
        return self.batch * self.seq

    @property
    def elements(self) -> int:
        return self.rows * self.d

    @property
    def d_g(self) -> int:
        return self.d // self.n_groups

    @property
    def io_bytes(self) -> int:
        return 2 if self.io == "bf16" else 4

    def with_rows(self, rows: int) -> "Workload":
        """Same recipe with `rows` rows in total (batch = rows, seq = 1)."""
        return replace(self, batch=rows, seq=1)


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny", 2, 8, 32, 8, "f32", 0.5, 1.0, 1.0, 1),
        Workload("kat-t", 128, 197, 192, 8, "f32", 0.5, 1.0, 1e-2, 2),
        Workload("kat-s-hid", 1024, 197, 1536, 8, "f32", 0.5, 1.0, 1e-2, 3, True),
        Workload("kat-b", 1024, 197, 768, 8, "f32", 0.5, 1.0, 1e-2, 4),
        Workload("kat-b-hid-bf16", 1024, 197, 3072, 8, "bf16", 0.5, 1.0, 1e-2, 5),
        Workload("kat-b-pau", 1024, 197, 768, 1, "f32", 0.5, 1.0, 1e-2, 6),
        Workload("kat-b-r32", 1024, 197, 768, 8, "f32", 0.5, 1.0, 1e-2, 7, m=3, n=2),
        Workload("kat-b-r76", 1024, 197, 768, 8, "f32", 0.5, 1.0, 1e-2, 8, m=7, n=6),
        Workload("kat-b-poly5", 1024, 197, 768, 8, "f32", 0.5, 1.0, 1e-2, 9, m=5, n=0),
        Workload("kat-b-perchan", 1024, 197, 768, 768, "f32", 0.5, 1.0, 1e-2, 10),
        Workload("kat-b-layer1-bf16", 1024, 197, 768, 8, "bf16", 0.5, 1.0, 1e-2, 11, d_out=3072),
        Workload("kat-b-layer2-bf16", 1024, 197, 3072, 8, "bf16", 0.5, 1.0, 1e-2, 12, d_out=768),
        Workload("kat-b-cheby-bf16", 1024, 197, 768, 1, "bf16", 0.5, 1.0, 1e-2, 13, d_out=768, cheby=7),
    )
}

# The GR-KAN workloads (degrees (5, 4), 8 groups) and the PAU-family ones.
GRKAN_WORKLOADS = ("tiny", "kat-t", "kat-s-hid", "kat-b", "kat-b-hid-bf16")
PAU_WORKLOADS = ("kat-b-pau", "kat-b-r32", "kat-b-r76", "kat-b-poly5", "kat-b-perchan")
LAYER_WORKLOADS = ("kat-b-layer1-bf16", "kat-b-layer2-bf16")
CHEBY_WORKLOADS = ("kat-b-cheby-bf16",)


def custom(name: str, rows: int, d: int, n_groups: int, m: int = 5, n: int = 4, io: str = "f32",
           seed: int = 100, coef_std: float = 0.5, dy_std: float = 1e-2, d_out: int = 0,
           cheby: int = 0) -> Workload:
    """A workload of the same recipe with any shape, group count and degrees."""
    return Workload(name, rows, 1, d, n_groups, io, coef_std, 1.0, dy_std, seed, m=m, n=n, d_out=d_out,
                    cheby=cheby)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest-even bf16; returns the uint16 bit patterns."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact float32 value of bf16 bit patterns (uint16)."""
    return (h.astype(np.uint32) << 16).view(np.float32)


def _draws(w: Workload):
    rng = np.random.default_rng(w.seed)
    std = np.float32(w.coef_std)
    A = rng.standard_normal((w.n_groups, w.m + 1), dtype=np.float32) * std
    B = rng.standard_normal((w.n_groups, w.n), dtype=np.float32) * std
    if w.identity_group0:
        A[0] = 0
        A[0, 1] = 1
    return rng, A.astype(np.float32), B.astype(np.float32)


def coefficients(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    _, A, B = _draws(w)
    return A, B


def weight(w: Workload) -> np.ndarray:
    """The layer's W [d_out, d] (Chebyshev: C [d_out, d, degree + 1]) as bf16 bit patterns."""
    if w.d_out <= 0:
        raise ValueError("not a layer workload")
    rng, _, _ = _draws(w)
    if w.cheby:
        nb = w.cheby + 1
        C = rng.standard_normal((w.d_out, w.d, nb), dtype=np.float32)
        C *= np.float32(1.0 / np.sqrt(w.d * nb))
        return bf16_bits(C).reshape(w.d_out, w.d, nb)
    W = rng.standard_normal((w.d_out, w.d), dtype=np.float32)
    W *= np.float32(1.0 / np.sqrt(w.d))
    return bf16_bits(W).reshape(w.d_out, w.d)


def _tensor(w: Workload, which: int, std: float, out: np.ndarray) -> None:
    """Fill the flat `out` (float32, or uint16 for bf16) with tensor `which`."""
    n = out.size
    nchunk = (n + CHUNK - 1) // CHUNK
    s = np.float32(std)

    def fill(k):
        lo, hi = k * CHUNK, min(n, (k + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed, spawn_key=(which, k))))
        if w.io == "bf16":
            tmp = g.standard_normal(hi - lo, dtype=np.float32)
            if std != 1.0:
                np.multiply(tmp, s, out=tmp)
            out[lo:hi] = bf16_bits(tmp)
        else:
            dst = out[lo:hi]
            g.standard_normal(out=dst, dtype=np.float32)
            if std != 1.0:
                np.multiply(dst, s, out=dst)

    if nchunk <= 1:
        for k in range(nchunk):
            fill(k)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunk)))


def make_inputs(w: Workload | str, rows: int | None = None, need_dy: bool = True) -> dict:
    """Inputs of workload `w` (optionally only its first `rows` rows).

    Returns ``{"A", "B", "x", "dy", "workload"}`` with x/dy shaped [rows, d]
    (float32, or uint16 bf16 bit patterns when ``w.io == "bf16"``); a layer
    workload has ``"W"`` [d_out, d] and, in place of dy, ``"dz"`` [rows, d_out].
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    if rows is not None:
        if rows > w.rows:
            raise ValueError("rows beyond the workload's size")
        w = w.with_rows(rows)
    A, B = coefficients(w)
    dt = np.uint16 if w.io == "bf16" else np.float32
    x = np.empty(w.elements, dtype=dt)
    _tensor(w, 1, w.x_std, x)
    dy = None
    if need_dy and w.d_out == 0:
        dy = np.empty(w.elements, dtype=dt)
        _tensor(w, 2, w.dy_std, dy)
        dy = dy.reshape(w.rows, w.d)
    out = {"A": A, "B": B, "x": x.reshape(w.rows, w.d), "dy": dy, "workload": w}
    if w.d_out > 0:
        out["W"] = weight(w)
        if need_dy:
            dz = np.empty(w.rows * w.d_out, dtype=dt)
            _tensor(w, 3, w.dy_std, dz)
            out["dz"] = dz.reshape(w.rows, w.d_out)
    return out
