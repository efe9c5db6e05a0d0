"""GPU parity of the Chebyshev-KAN layer (grkan_chebykan_forward / _backward,
the case study of "PolyKAN: Efficient Fused GPU Operators for Polynomial
Kolmogorov-Arnold Network Variants", abstract page) against the fp64 oracle
(oracle/chebykan.py): several 256 x 256 tiles with ragged rows and columns,
row splits of the coefficient gradient, special inputs (zeros, saturating
|x|, the tanh switch point), the empty case, and the full-size workload on
sampled rows and coefficient entries.
"""
import math
import sys

import numpy as np
import pytest
import torch

from gr_kan_rational_amd import synth
from oracle import chebykan as ck
from oracle import layer
from oracle import oracle as orc
import parity

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
D = 7


@pytest.fixture(scope="module")
def gk():
    import gr_kan_rational_amd.binding as b

    b.load_library()
    return b


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def inputs(rows, d_in, d_out, seed):
    w = synth.custom("cheby", rows, d_in, 1, io="bf16", seed=seed, d_out=d_out, cheby=D)
    return synth.make_inputs(w)


def check_forward(name, y, ref, k):
    parity.check_layer(name, y, {"z": ref["y"], "amb": ref["amb"], "mag": ref["mag"]}, k)


def check_dx(name, dx, ref):
    tol = ref["dxerr"] + 0.5 * parity.ulp_bf16(dx)
    err = np.abs(dx - ref["dx"])
    bad = err > tol
    if bad.any():
        i = int(np.flatnonzero(bad.ravel())[0])
        raise AssertionError(f"{name}: {int(bad.sum())} of {dx.size} outside tolerance; first at {i}: "
                             f"gpu {dx.ravel()[i]!r} ref {ref['dx'].ravel()[i]!r} tol {tol.ravel()[i]!r}")


# (rows, d_in, d_out)
SHAPES = [(301, 64, 300), (257, 256, 512), (700, 96, 128), (33, 8, 64), (3000, 32, 64)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_chebykan_parity(gk, shape):
    rows, d_in, d_out = shape
    log(f"[cheby] rows={rows} d_in={d_in} d_out={d_out}")
    inp = inputs(rows, d_in, d_out, 8000 + rows)
    inp["x"][::7, ::3] = 0
    x, C, dy = bf(inp["x"]), bf(inp["W"]), bf(inp["dz"])
    y = gk.grkan_chebykan_forward(x, C)
    torch.cuda.synchronize()
    check_forward(f"cheby y {shape}", host(y), ck.forward(inp["x"], inp["W"], D), d_in * (D + 1))
    if d_out % 64 == 0:
        dx, dC = gk.grkan_chebykan_backward(x, dy, C)
        dx2, dC2 = gk.grkan_chebykan_backward(x, dy, C)
        torch.cuda.synchronize()
        ref = ck.backward(inp["x"], inp["dz"], inp["W"], D)
        check_dx(f"cheby dx {shape}", host(dx), ref)
        parity.check_sums(f"cheby dC {shape}", dC.cpu().numpy(), ref["dC"], ref["dC_norm"], extra=ref["dC_amb"])
        assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16)) and torch.equal(dC, dC2)


def test_chebykan_special_inputs(gk):
    """x = 0 (t = 0), |x| large (t = +-1), and x on both sides of the point where the tanh
    evaluation switches from its series to the exponential form."""
    rows, d_in, d_out = 64, 64, 64
    inp = inputs(rows, d_in, d_out, 8100)
    vals = np.float32([0.0, -0.0, 9.0, -9.0, 40.0, -100.0, 0.546875, 0.5546875, -0.546875, -0.5546875,
                       1e-3, -1e-30, 3.0, 0.25, 1.0, -2.0])
    inp["x"][:, :16] = synth.bf16_bits(np.tile(vals, (rows, 1)))
    x, C, dy = bf(inp["x"]), bf(inp["W"]), bf(inp["dz"])
    y = gk.grkan_chebykan_forward(x, C)
    dx, dC = gk.grkan_chebykan_backward(x, dy, C)
    torch.cuda.synchronize()
    check_forward("cheby special y", host(y), ck.forward(inp["x"], inp["W"], D), d_in * (D + 1))
    ref = ck.backward(inp["x"], inp["dz"], inp["W"], D)
    check_dx("cheby special dx", host(dx), ref)
    parity.check_sums("cheby special dC", dC.cpu().numpy(), ref["dC"], ref["dC_norm"], extra=ref["dC_amb"])


def test_chebykan_in_place_and_empty(gk):
    inp = inputs(100, 64, 64, 8200)
    x, C, dy = bf(inp["x"]), bf(inp["W"]), bf(inp["dz"])
    dx, dC = gk.grkan_chebykan_backward(x, dy, C)
    xc = x.clone()
    dx2, _ = gk.grkan_chebykan_backward(xc, dy, C, dx=xc)
    dC0 = torch.full_like(dC, 3.0)
    gk.grkan_chebykan_backward(x[:0], dy[:0], C, dC=dC0)
    y0 = gk.grkan_chebykan_forward(x[:0], C)
    torch.cuda.synchronize()
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16))
    assert not dC0.any() and y0.shape == (0, 64)


def test_chebykan_rejects(gk):
    inp = inputs(4, 64, 64, 8300)
    with pytest.raises(gk.GRKANError) as e:
        gk.grkan_chebykan_forward(bf(inp["x"]), bf(inp["W"])[:, :, :4].contiguous(), degree=3)
    assert e.value.status == gk.GRKAN_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", list(synth.CHEBY_WORKLOADS))
def test_chebykan_full_size_sampled(gk, name):
    """Full size, in the benchmark's configuration: y and dx on sampled rows, dC on sampled
    entries (one coefficient column of the basis over all rows), against the oracle."""
    w = synth.WORKLOADS[name]
    log(f"[cheby_full] {name}")
    inp = synth.make_inputs(w)
    x, C, dy = bf(inp["x"]), bf(inp["W"]), bf(inp["dz"])
    y = gk.grkan_chebykan_forward(x, C)
    dx, dC = gk.grkan_chebykan_backward(x, dy, C)
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    rows = np.unique(np.concatenate([[0, w.rows - 1], rng.integers(0, w.rows, 30)]))
    sel = torch.from_numpy(rows).to(DEV)
    check_forward(f"{name} y rows", host(y[sel]), ck.forward(inp["x"][rows], inp["W"], D), w.d * (D + 1))
    ref = ck.backward(inp["x"][rows], inp["dz"][rows], inp["W"], D)
    check_dx(f"{name} dx rows", host(dx[sel]), ref)
    dCh = dC.cpu().numpy()
    dyv = orc.to_f64(inp["dz"], "bf16")
    for o, i in zip(rng.integers(0, w.d_out, 8), rng.integers(0, w.d, 8)):
        xi = orc.to_f64(inp["x"][:, i], "bf16")
        T = ck.chebyshev_t(np.tanh(xi), D)
        err = ck.basis_error(np.arange(D + 1))
        Tb = layer.bf16_round(T)
        lo, hi = layer.bf16_round(T - err), layer.bf16_round(T + err)
        width = np.where(lo != hi, hi - lo, 0.0)
        for k in range(D + 1):
            terms = dyv[:, o] * Tb[:, k]
            refv = math.fsum(terms)
            amb = float(np.sum(np.abs(dyv[:, o]) * width[:, k]))
            norm = float(np.sqrt(np.sum(terms * terms)))
            parity.check_sums(f"{name} dC[{o},{i},{k}]", np.array([dCh[o, i, k]]), np.array([refv]),
                              np.array([norm]), extra=np.array([amb]))
