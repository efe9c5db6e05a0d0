"""GPU parity of the PAU family (other degrees (m, n) and group counts) against
the fp64 oracle, through the grkan_pau_* C ABI.

The pages note that the kernel restructuring applies to PAU and its variants
([FlashKAT notes], section "局限性与未来工作"); these tests cover every degree
pair the library compiles, both I/O types, one shared function (n_g = 1),
groups whose row segment is split into several ragged column parts, ragged
row tails, and the full-size PAU workloads in the benchmark's launch
configuration.  Tolerances: tests/parity.py.
"""
import json
import os
import sys

import numpy as np
import pytest
import torch

from gr_kan_rational_amd import synth
from oracle import oracle as orc
import nearroot
import parity

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PAIRS = [(5, 4), (3, 2), (4, 3), (6, 5), (7, 6), (2, 1), (4, 4), (5, 0)]
# (rows, d, n_groups): 32-channel groups; one group of 768 channels; two groups of 4000
# channels (16000 / 8000 bytes per row segment: 3 to 6 ragged column parts)
GEOMS = [(301, 256, 8), (203, 768, 1), (37, 8000, 2)]


@pytest.fixture(scope="module")
def gk():
    import gr_kan_rational_amd.binding as b

    b.load_library()
    return b


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, io):
    if io == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t, io):
    return t.float().cpu().numpy() if io == "bf16" else t.cpu().numpy()


def coef_dev(inp):
    A = torch.from_numpy(inp["A"]).to(DEV)
    B = torch.from_numpy(inp["B"]).to(DEV) if inp["B"].size else None
    return A, B


def iocode(gk, io):
    return gk.GRKAN_BF16 if io == "bf16" else gk.GRKAN_F32


def run_and_check(gk, w, inp, mode, tag):
    m, n = w.m, w.n
    x, dy = to_dev(inp["x"], w.io), to_dev(inp["dy"], w.io)
    A, B = coef_dev(inp)
    y = gk.grkan_pau_forward(x, A, B, w.n_groups, m, n)
    dx, dA, dB = gk.grkan_pau_backward(x, dy, A, B, w.n_groups, m, n, mode=mode)
    torch.cuda.synchronize()
    ref = orc.run(inp["x"], inp["A"], inp["B"], w.n_groups, dy=inp["dy"], io=w.io, m=m, n=n)
    n_add = 0
    if mode == "block_atomic":
        n_add = gk.grkan_pau_query_launch(w.rows, w.d, w.n_groups, m, n, iocode(gk, w.io), 2)["tiles"]
        n_add *= gk.grkan_pau_query_launch(w.rows, w.d, w.n_groups, m, n, iocode(gk, w.io), 2)["parts"]
    parity.check_elem(f"{tag} Y", to_host(y, w.io), ref["y"], ref["ymag"], w.io)
    parity.check_elem(f"{tag} dX", to_host(dx, w.io), ref["dx"], ref["dxmag"], w.io)
    parity.check_sums(f"{tag} dA", dA.cpu().numpy(), ref["dA"], ref["nA"], n_add,
                      parity.term_mag(m, n, ref["mA"]))
    if n > 0:
        parity.check_sums(f"{tag} dB", dB.cpu().numpy(), ref["dB"], ref["nB"], n_add,
                          parity.term_mag(m, n, ref["mB"]))
    else:
        assert dB is None


@pytest.mark.parametrize("m,n", PAIRS)
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("geom", GEOMS, ids=lambda g: f"{g[0]}x{g[1]}g{g[2]}")
def test_pau_parity(gk, m, n, io, geom):
    rows, d, n_g = geom
    w = synth.custom(f"pau{m}{n}", rows, d, n_g, m=m, n=n, io=io, seed=1000 + 10 * m + n)
    log(f"[pau_parity] (m,n)=({m},{n}) io={io} rows={rows} d={d} n_g={n_g}")
    inp = synth.make_inputs(w)
    run_and_check(gk, w, inp, "deterministic", f"({m},{n}) {io} {geom}")


# Narrow groups (row segments that are not whole 16-byte vectors): one PAU per channel, 5-channel
# groups, 3-channel groups, 125-channel groups spanning up to 3 column blocks of 64 channels,
# an odd channel count (bf16 rows that are not whole 4-byte words), and 5-channel groups over
# several whole 256-row backward tiles and a ragged tail.
NARROW = [(301, 768, 768), (203, 40, 8), (129, 300, 100), (97, 1000, 8), (67, 99, 33), (1100, 200, 40)]


@pytest.mark.parametrize("m,n", [(5, 4), (3, 2), (7, 6), (5, 0), (2, 1)])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("geom", NARROW, ids=lambda g: f"{g[0]}x{g[1]}g{g[2]}")
def test_pau_parity_narrow(gk, m, n, io, geom):
    rows, d, n_g = geom
    w = synth.custom(f"narrow{m}{n}", rows, d, n_g, m=m, n=n, io=io, seed=3000 + 10 * m + n)
    log(f"[pau_narrow] (m,n)=({m},{n}) io={io} rows={rows} d={d} n_g={n_g}")
    inp = synth.make_inputs(w)
    run_and_check(gk, w, inp, "deterministic", f"narrow ({m},{n}) {io} {geom}")


@pytest.mark.parametrize("geom", NARROW[:3], ids=lambda g: f"{g[0]}x{g[1]}g{g[2]}")
def test_pau_parity_narrow_block_atomic(gk, geom):
    rows, d, n_g = geom
    w = synth.custom("narrow54a", rows, d, n_g, m=5, n=4, io="f32", seed=4000 + n_g)
    log(f"[pau_narrow_block_atomic] rows={rows} d={d} n_g={n_g}")
    run_and_check(gk, w, synth.make_inputs(w), "block_atomic", f"narrow block_atomic {geom}")


def test_narrow_special_values(gk):
    """One PAU per channel with exact zeros, b = 0 channels and x at a root of Q: the narrow
    kernel's sign-fix path, element by element against the oracle."""
    w = synth.custom("narrowspecial", 96, 64, 64, m=3, n=2, io="f32", seed=77)
    inp = synth.make_inputs(w)
    inp["x"][::3, :] = 0.0                    # exact zeros: s = 0
    inp["B"][5] = 0.0                         # a channel with Q identically 0
    inp["B"][7] = np.array([-0.75, 1.0], np.float32)   # Q = x (x - 0.75): root at 0.75
    inp["x"][1::3, 7] = np.float32(0.75)
    run_and_check(gk, w, inp, "deterministic", "narrow special values")


# (rows, d, n_groups): 8-channel groups (the segment kernels, a small grid), one function
# per channel (the narrow kernels), and 96-channel groups on a grid large enough for the
# kernels the full-size workloads run
NEAR_ROOT_GEOMS = [(96, 64, 8), (96, 64, 64), (65536, 768, 8)]


@pytest.mark.parametrize("m,n", [(7, 6), (6, 5), (5, 4)])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("geom", NEAR_ROOT_GEOMS, ids=lambda g: f"{g[0]}x{g[1]}g{g[2]}")
def test_exact_sign_at_clustered_roots(gk, m, n, io, geom):
    """x next to 3- to 5-fold roots of q (tests/nearroot.py), where the sign of Q lies below
    fp64's resolution and compensated Horner's: every unproven element's sign must be the
    oracle's exact one.  A wrong sign moves that element's dB terms by 2 |v x^j|, far beyond
    the sums' tolerance; dX moves little there (Q' vanishes at a multiple root)."""
    rows, d, n_g = geom
    inp = nearroot.make(m, n, n_g, d, rows, seed=100 * m + n, io=io)
    w = synth.custom(f"nearroot{m}{n}", rows, d, n_g, m=m, n=n, io=io, seed=0)
    for mode in ("deterministic", "block_atomic"):
        log(f"[exact_sign] (m,n)=({m},{n}) io={io} rows={rows} d={d} n_g={n_g} {mode}")
        run_and_check(gk, w, inp, mode, f"clustered roots ({m},{n}) {io} {geom} {mode}")


@pytest.mark.parametrize("m,n", [(5, 4), (3, 2), (7, 6), (5, 0)])
@pytest.mark.parametrize("geom", GEOMS, ids=lambda g: f"{g[0]}x{g[1]}g{g[2]}")
def test_pau_parity_block_atomic(gk, m, n, geom):
    rows, d, n_g = geom
    w = synth.custom(f"pau{m}{n}", rows, d, n_g, m=m, n=n, io="f32", seed=2000 + 10 * m + n)
    log(f"[pau_block_atomic] (m,n)=({m},{n}) rows={rows} d={d} n_g={n_g}")
    run_and_check(gk, w, synth.make_inputs(w), "block_atomic", f"({m},{n}) block_atomic {geom}")


def test_pau_54_is_grkan_bitwise(gk):
    """grkan_pau_* at (5, 4) and the GR-KAN entry points run the same kernels."""
    inp = synth.make_inputs("kat-b", rows=257)
    w = inp["workload"]
    x, dy = to_dev(inp["x"], "f32"), to_dev(inp["dy"], "f32")
    A, B = coef_dev(inp)
    y1 = gk.grkan_forward(x, A, B, 8)
    y2 = gk.grkan_pau_forward(x, A, B, 8, 5, 4)
    r1 = gk.grkan_backward(x, dy, A, B, 8)
    r2 = gk.grkan_pau_backward(x, dy, A, B, 8, 5, 4)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    assert w.rows == 257


def test_pau_empty_and_b_zero(gk):
    """rows == 0 writes zero sums; a (3, 2) group with b = 0 takes the Q == 0 path (s = 0)."""
    A = torch.randn(4, 4, device=DEV)
    B = torch.randn(4, 2, device=DEV)
    x = torch.empty(0, 64, device=DEV)
    _, dA, dB = gk.grkan_pau_backward(x, x, A, B, 4, 3, 2)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dA) == 0 and torch.count_nonzero(dB) == 0
    w = synth.custom("bzero", 129, 64, 4, m=3, n=2, seed=77)
    inp = synth.make_inputs(w)
    inp["B"][1] = 0.0
    inp["A"][2] = np.array([0, 1, 0, 0], np.float32)
    inp["B"][2] = 0.0
    run_and_check(gk, w, inp, "deterministic", "(3,2) b=0 groups")


@pytest.mark.parametrize("name", list(synth.PAU_WORKLOADS))
def test_pau_full_size(gk, name):
    """Full-size PAU workloads: sampled elements one by one, and the full group sums."""
    w = synth.WORKLOADS[name]
    m, n = w.m, w.n
    log(f"[pau_full] {name} shape=({w.batch},{w.seq},{w.d}) n_g={w.n_groups} (m,n)=({m},{n})")
    inp = synth.make_inputs(w)
    x, dy = to_dev(inp["x"], w.io), to_dev(inp["dy"], w.io)
    A, B = coef_dev(inp)
    y = gk.grkan_pau_forward(x, A, B, w.n_groups, m, n)
    dx, dA, dB = gk.grkan_pau_backward(x, dy, A, B, w.n_groups, m, n)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    idx = np.unique(np.concatenate([rng.integers(0, w.elements, 200_000, dtype=np.int64),
                                    np.arange(2 * w.d, dtype=np.int64),
                                    np.arange(w.elements - 2 * w.d, w.elements, dtype=np.int64)]))
    it = torch.from_numpy(idx).to(DEV)
    ys = to_host(y.reshape(-1).index_select(0, it), w.io)
    dxs = to_host(dx.reshape(-1).index_select(0, it), w.io)
    del x, dy, y, dx
    rec = orc.points(inp["x"], inp["A"], inp["B"], w.n_groups, idx, dy=inp["dy"], io=w.io, m=m, n=n)
    parity.check_elem(f"{name} Y[sampled]", ys, rec[:, orc.F], rec[:, orc.FMAG], w.io)
    parity.check_elem(f"{name} dX[sampled]", dxs, rec[:, orc.DX], rec[:, orc.DXMAG], w.io)
    g = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                    f"{name}.sums.json")))
    parity.check_sums(f"{name} dA", dA.cpu().numpy(), np.array(g["dA"]), np.array(g["nA"]),
                      mag=parity.term_mag(m, n, np.array(g["mA"])))
    if n > 0:
        parity.check_sums(f"{name} dB", dB.cpu().numpy(), np.array(g["dB"]), np.array(g["nB"]),
                          mag=parity.term_mag(m, n, np.array(g["mB"])))
    log(f"[pau_full] {name}: ok")
