"""The C-ABI calls under HIP graph capture: the library allocates nothing,
sets no memory with memset nodes (dA/dB and dW/dC are cleared or written by
kernels) and never synchronises, so a forward + backward sequence can be
captured once and replayed.  Each test warms the calls up eagerly, captures
them into a torch.cuda.CUDAGraph with preallocated outputs and workspaces,
then replays the graph several times with new inputs copied in eagerly
between replays (and other eager work on the same buffers), and checks every
replay bit for bit against the same calls made eagerly on the same inputs.
The block-atomic backward's dA/dB depend on the order of the atomics, so
there only dx is compared bit for bit and dA/dB within the sum rule.
"""
import sys

import numpy as np
import pytest
import torch

from gr_kan_rational_amd import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REPLAYS = 3


@pytest.fixture(scope="module")
def gk():
    import gr_kan_rational_amd.binding as b

    b.load_library()
    return b


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t.view(dtype) if dtype is not None else t


def capture(fn):
    """fn() captured once after an eager warm-up on a side stream (torch's capture protocol)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("mode", ["deterministic", "block_atomic"])
def test_activation_forward_backward_replays(gk, mode):
    w = synth.custom("graph", 4000, 192, 8, io="f32", seed=901)
    log(f"[graph activation] mode={mode} rows={w.rows} d={w.d}")
    inp = synth.make_inputs(w)
    x, dy = dev(inp["x"]).view(torch.float32), dev(inp["dy"]).view(torch.float32)
    A, B = dev(inp["A"]), dev(inp["B"])
    y, dx = torch.empty_like(x), torch.empty_like(x)
    dA, dB = torch.empty((8, 6), device=DEV), torch.empty((8, 4), device=DEV)
    ws = torch.empty(max(1, gk.grkan_backward_workspace_size(w.rows, w.d, 8, gk.GRKAN_F32,
                                                             gk._MODES[mode])), dtype=torch.uint8, device=DEV)

    def step():
        gk.grkan_forward(x, A, B, 8, out=y)
        gk.grkan_backward(x, dy, A, B, 8, mode=mode, dx=dx, dA=dA, dB=dB, workspace=ws)

    g = capture(step)
    for rep in range(REPLAYS):
        fresh = synth.make_inputs(synth.custom("graph", w.rows, w.d, 8, io="f32", seed=910 + rep))
        x.copy_(dev(fresh["x"]).view(torch.float32))
        dy.copy_(dev(fresh["dy"]).view(torch.float32))
        dx.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (y, dx, dA, dB)]
        y.zero_()
        step()                                   # eager, same inputs, same buffers
        torch.cuda.synchronize()
        assert torch.equal(got[0], y) and torch.equal(got[1], dx), f"replay {rep}: y/dx differ"
        if mode == "deterministic":
            assert torch.equal(got[2], dA) and torch.equal(got[3], dB), f"replay {rep}: dA/dB differ"
        else:
            for a, b in ((got[2], dA), (got[3], dB)):
                assert torch.allclose(a, b, rtol=1e-4, atol=1e-6), f"replay {rep}: atomic sums differ"


def test_layer_forward_backward_replays(gk):
    rows, d_in, d_out, n_g = 300, 256, 320, 8
    log(f"[graph layer] rows={rows} d_in={d_in} d_out={d_out}")
    w = synth.custom("graph-layer", rows, d_in, n_g, io="bf16", seed=920, d_out=d_out)
    inp = synth.make_inputs(w)
    x, dz, W = (dev(inp[k].view(np.int16)).view(torch.bfloat16) for k in ("x", "dz", "W"))
    A, B = dev(inp["A"]), dev(inp["B"])
    z = torch.empty((rows, d_out), dtype=torch.bfloat16, device=DEV)
    dx = torch.empty_like(x)
    dA, dB = torch.empty((n_g, 6), device=DEV), torch.empty((n_g, 4), device=DEV)
    dW = torch.empty((d_out, d_in), device=DEV)
    ws = torch.empty(gk.grkan_layer_backward_workspace_size(rows, d_in, d_out, n_g), dtype=torch.uint8, device=DEV)

    def step():
        gk.grkan_layer_forward(x, A, B, W, n_g, out=z)
        gk.grkan_layer_backward(x, dz, A, B, W, n_g, dx=dx, dA=dA, dB=dB, dW=dW, workspace=ws)

    g = capture(step)
    for rep in range(REPLAYS):
        fresh = synth.make_inputs(synth.custom("graph-layer", rows, d_in, n_g, io="bf16", seed=930 + rep,
                                               d_out=d_out))
        x.copy_(dev(fresh["x"].view(np.int16)).view(torch.bfloat16))
        dz.copy_(dev(fresh["dz"].view(np.int16)).view(torch.bfloat16))
        dW.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (z, dx, dA, dB, dW)]
        step()
        torch.cuda.synchronize()
        for name, a, b in zip(("z", "dx", "dA", "dB", "dW"), got, (z, dx, dA, dB, dW)):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"


def test_chebykan_forward_backward_replays(gk):
    rows, d_in, d_out = 300, 64, 128
    log(f"[graph cheby] rows={rows} d_in={d_in} d_out={d_out}")
    w = synth.custom("graph-cheby", rows, d_in, 1, io="bf16", seed=940, d_out=d_out, cheby=7)
    inp = synth.make_inputs(w)
    x = dev(inp["x"].view(np.int16)).view(torch.bfloat16)
    dy = dev(inp["dz"].view(np.int16)).view(torch.bfloat16)
    C = dev(inp["W"].view(np.int16)).view(torch.bfloat16).view(d_out, d_in, 8)
    y = torch.empty((rows, d_out), dtype=torch.bfloat16, device=DEV)
    dx = torch.empty_like(x)
    dC = torch.empty((d_out, d_in, 8), device=DEV)
    ws = torch.empty(gk.grkan_chebykan_backward_workspace_size(rows, d_in, d_out), dtype=torch.uint8, device=DEV)

    def step():
        gk.grkan_chebykan_forward(x, C, out=y)
        gk.grkan_chebykan_backward(x, dy, C, dx=dx, dC=dC, workspace=ws)

    g = capture(step)
    for rep in range(REPLAYS):
        fresh = synth.make_inputs(synth.custom("graph-cheby", rows, d_in, 1, io="bf16", seed=950 + rep,
                                               d_out=d_out, cheby=7))
        x.copy_(dev(fresh["x"].view(np.int16)).view(torch.bfloat16))
        dy.copy_(dev(fresh["dz"].view(np.int16)).view(torch.bfloat16))
        dC.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (y, dx, dC)]
        step()
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "dx", "dC"), got, (y, dx, dC)):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
