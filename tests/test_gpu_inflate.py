"""GPU checks of the FLOP-inflation probe (grkan_inflated_forward /
grkan_inflated_backward): the pages' Insight 2 ([FlashKAT notes], section
"1. 性能瓶颈诊断") multiplies the rational's arithmetic by 8 and watches the
run time.  The probe must change only the arithmetic: its outputs are those of
grkan_forward / grkan_backward bit for bit (same kernels' memory traffic, same
reduction order), for every repeat count, both I/O types, ragged tiles and
column parts, b = 0 groups (the Q = 0 variant), exact zeros and x at a root of
Q (the sign-fix path), and at full workload size; and they match the fp64
oracle within the tolerances of tests/parity.py.
"""
import sys

import numpy as np
import pytest
import torch

from gr_kan_rational_amd import synth
from oracle import oracle as orc
import parity

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REPEATS = [2, 4, 8]
GEOMS = [(301, 256, 8), (203, 768, 8), (37, 8000, 2)]


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


def special(inp, n_g, d):
    """Exact zeros, a b = 0 group and x at a root of Q in another group."""
    d_g = d // n_g
    inp["x"][:, ::5] = 0
    inp["B"][n_g - 1] = 0.0
    inp["B"][0] = np.array([-0.75, 1.0, 0.0, 0.0], np.float32)   # Q = x (x - 0.75)
    v = np.float32(0.75)
    inp["x"][1::7, :d_g:3] = synth.bf16_bits(np.array([v]))[0] if inp["x"].dtype == np.uint16 else v
    return inp


def bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def plain_and_inflated(gk, w, inp, repeat, mode="deterministic"):
    x, dy = to_dev(inp["x"], w.io), to_dev(inp["dy"], w.io)
    A, B = torch.from_numpy(inp["A"]).to(DEV), torch.from_numpy(inp["B"]).to(DEV)
    y0 = gk.grkan_forward(x, A, B, w.n_groups)
    y1 = gk.grkan_inflated_forward(x, A, B, w.n_groups, repeat=repeat)
    g0 = gk.grkan_backward(x, dy, A, B, w.n_groups, mode=mode)
    g1 = gk.grkan_inflated_backward(x, dy, A, B, w.n_groups, repeat=repeat, mode=mode)
    torch.cuda.synchronize()
    return (y0, *g0), (y1, *g1)


@pytest.mark.parametrize("repeat", REPEATS)
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("geom", GEOMS, ids=lambda g: f"{g[0]}x{g[1]}g{g[2]}")
def test_inflated_equals_plain_bitwise(gk, repeat, io, geom):
    rows, d, n_g = geom
    w = synth.custom("inflate", rows, d, n_g, io=io, seed=5000 + rows)
    log(f"[inflate_bitwise] repeat={repeat} io={io} rows={rows} d={d} n_g={n_g}")
    inp = special(synth.make_inputs(w), n_g, d)
    plain, infl = plain_and_inflated(gk, w, inp, repeat)
    for name, a, b in zip(("y", "dx", "dA", "dB"), plain, infl):
        assert np.array_equal(bits(a), bits(b)), f"{name} differs at repeat {repeat}"


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["deterministic", "block_atomic"])
def test_inflated_parity_vs_oracle(gk, io, mode):
    w = synth.custom("inflate_orc", 301, 256, 8, io=io, seed=5100)
    log(f"[inflate_oracle] repeat=8 io={io} mode={mode}")
    inp = special(synth.make_inputs(w), 8, 256)
    _, (y, dx, dA, dB) = plain_and_inflated(gk, w, inp, 8, mode)
    ref = orc.run(inp["x"], inp["A"], inp["B"], 8, dy=inp["dy"], io=io)
    n_add = 0
    if mode == "block_atomic":
        q = gk.grkan_query_launch(w.rows, w.d, 8, gk.GRKAN_BF16 if io == "bf16" else gk.GRKAN_F32, 2)
        n_add = q["tiles"] * q["parts"]
    parity.check_elem("inflated Y", to_host(y, io), ref["y"], ref["ymag"], io)
    parity.check_elem("inflated dX", to_host(dx, io), ref["dx"], ref["dxmag"], io)
    parity.check_sums("inflated dA", dA.cpu().numpy(), ref["dA"], ref["nA"], n_add)
    parity.check_sums("inflated dB", dB.cpu().numpy(), ref["dB"], ref["nB"], n_add)


@pytest.mark.parametrize("name", ["kat-b", "kat-b-hid-bf16"])
def test_inflated_full_size_bitwise(gk, name):
    """At full workload size, in the benchmark's launch configuration, repeat = 8 gives the
    plain outputs bit for bit (the plain path's parity is checked against the oracle in
    test_gpu_parity.py)."""
    w = synth.WORKLOADS[name]
    log(f"[inflate_full] {name} repeat=8")
    plain, infl = plain_and_inflated(gk, w, synth.make_inputs(w), 8)
    for nm, a, b in zip(("y", "dx", "dA", "dB"), plain, infl):
        it = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a.view(it), b.view(it)), f"{nm} differs at {name}"
