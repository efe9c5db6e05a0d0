"""Inputs next to clustered roots of q(x) = b_1 + b_2 x + ... + b_n x^(n-1).

Near a k-fold root r of q, |q(x)| falls like |x - r|^k while the terms b_j x^(j-1)
stay of order one, so the sign of Q = x q(x) at the fp32 neighbours of r is set
by bits far below fp64's (about 2^-123 of the terms for a 5-fold root at 2.75):
the backward must decide it exactly.  The roots are short binary fractions, so
that the expanded coefficients are exact in fp32 and the clusters stay exact
multiple roots.  Shared by the host test of the kernels' sign routine and the
GPU parity tests; holds none of the method's arithmetic.
"""
from fractions import Fraction

import numpy as np

# Root sets per denominator degree n (q has degree n - 1).
CLUSTERS = {
    6: [[2.75] * 5, [2.625] * 5, [-2.75] * 5, [2.75, 2.75, 2.75, 3.0, 3.0], [1.5, 1.5, 1.75, 1.75, 2.0],
        [0.75] * 5, [3.0] * 5, [-1.25] * 5],
    5: [[2.75] * 4, [2.625] * 4, [-3.0] * 4, [1.5, 1.5, 1.75, 1.75], [0.75] * 4, [2.75, 2.75, 3.0, 3.0],
        [-1.25] * 4, [2.5] * 4],
    4: [[2.75] * 3, [2.625] * 3, [-3.0] * 3, [1.5, 1.5, 1.75], [0.75] * 3, [2.5] * 3, [-1.25] * 3,
        [3.0] * 3],
}


def coefficients(roots):
    """Ascending coefficients b_1..b_n of prod (x - r), exactly, as fp32 (checked exact)."""
    c = [Fraction(1)]
    for r in roots:
        r = Fraction(r)
        nxt = [Fraction(0)] * (len(c) + 1)
        for i, a in enumerate(c):
            nxt[i + 1] += a
            nxt[i] -= a * r
        c = nxt
    out = np.array([float(v) for v in c], np.float32)
    assert all(Fraction(float(o)) == v for o, v in zip(out, c)), roots
    return out


def neighbours(r, k, dtype=np.float32):
    """The 2k + 1 values of `dtype` nearest to r (r itself included)."""
    if dtype == np.float32:
        v = np.float32(r)
        lo = [v]
        for _ in range(k):
            lo.append(np.nextafter(lo[-1], np.float32(-np.inf)))
        hi = [v]
        for _ in range(k):
            hi.append(np.nextafter(hi[-1], np.float32(np.inf)))
        return np.array(lo[::-1] + hi[1:], np.float32)
    # bf16 neighbours (r must be a bf16 value), returned as fp32 values: bf16 is
    # the top half of the fp32 bits
    bits = int(np.array([r], np.float32).view(np.uint32)[0]) >> 16
    return np.array([(bits + s) << 16 for s in range(-k, k + 1)], np.uint32).view(np.float32)


def make(m, n, n_g, d, rows, seed, io="f32", k=40):
    """x (rows, d), dy, A (n_g, m + 1), B (n_g, n): group g takes cluster g mod 8 of CLUSTERS[n];
    in every group's channels, even rows hold neighbours of the cluster's roots, row 1 exact
    zeros and tiny values, the other odd rows standard normal values.  bf16 x and dy come as uint16 bit patterns (dy rounded toward
    zero: any bf16 values will do)."""
    rng = np.random.default_rng(seed)
    sets = CLUSTERS[n]
    A = (rng.standard_normal((n_g, m + 1)) * 0.5).astype(np.float32)
    B = np.stack([coefficients(sets[g % len(sets)]) for g in range(n_g)])
    x = rng.standard_normal((rows, d)).astype(np.float32)
    dy = rng.standard_normal((rows, d)).astype(np.float32)
    d_g = d // n_g
    for g in range(n_g):
        roots = sorted(set(sets[g % len(sets)]))
        pool = np.concatenate([neighbours(r, k, np.float32 if io == "f32" else "bf16") for r in roots])
        cols = slice(g * d_g, (g + 1) * d_g)
        block = x[::2, cols]
        block[...] = pool[rng.integers(0, pool.size, block.shape)]
        x[::2, cols] = block
    # row 1: exact zeros (s = 0) and tiny x, whose terms span more bits than the kernels'
    # integer window holds (the sign then comes from the fp64 Q, here clear of rounding)
    specials = np.array([0.0, -0.0, 1e-30, -1e-30, 1e-20, -1e-20, 3e-12, -2e-9], np.float32)
    if rows > 1:
        x[1, :] = specials[np.arange(d) % specials.size]
    if io == "bf16":
        x = (x.view(np.uint32) >> 16).astype(np.uint16)
        dy = (dy.view(np.uint32) >> 16).astype(np.uint16)
    return {"x": x, "dy": dy, "A": A, "B": B}
