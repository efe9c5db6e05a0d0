"""GPU parity of the GR-KAN layer z = F(x) W^T (grkan_layer_forward: F fused
into the matrix-core GEMM) and of the plain GEMM (grkan_linear_forward)
against the fp64 layer oracle (oracle/layer.py), tolerances in
tests/parity.py.  Shapes span several 256 x 256 tiles with ragged row and
column tails, 8 to 64 groups, and the two KAT-B MLP layers at full size
(sampled rows).  The fused layer must equal the unfused composition
grkan_forward -> grkan_linear_forward bit for bit: both round the same fp32
F to bf16 and run the same matrix kernel.
"""
import math
import sys

import numpy as np
import pytest
import torch

from gr_kan_rational_amd import synth
from oracle import layer
from oracle import oracle as orc
import parity

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
# (rows, d_in, n_groups, d_out)
SHAPES = [(301, 256, 8, 272), (257, 768, 8, 3072), (300, 3072, 8, 768), (513, 512, 64, 256),
          (64, 128, 16, 48), (1, 64, 8, 1), (700, 1536, 24, 520)]


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


def inputs(rows, d_in, n_g, d_out, seed):
    w = synth.custom("layer", rows, d_in, n_g, io="bf16", seed=seed, d_out=d_out)
    return synth.make_inputs(w, need_dy=False)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_layer_parity(gk, shape):
    rows, d_in, n_g, d_out = shape
    log(f"[layer] rows={rows} d_in={d_in} n_g={n_g} d_out={d_out}")
    inp = inputs(rows, d_in, n_g, d_out, 6000 + rows)
    x, W = bf(inp["x"]), bf(inp["W"])
    A, B = torch.from_numpy(inp["A"]).to(DEV), torch.from_numpy(inp["B"]).to(DEV)
    z = gk.grkan_layer_forward(x, A, B, W, n_g)
    y = gk.grkan_forward(x, A, B, n_g)
    z2 = gk.grkan_linear_forward(y, W)
    torch.cuda.synchronize()
    ref = layer.forward(inp["x"], inp["A"], inp["B"], inp["W"], n_g)
    parity.check_layer(f"layer {shape}", host(z), ref, d_in)
    assert torch.equal(z.view(torch.int16), z2.view(torch.int16)), "fused and unfused differ"


@pytest.mark.parametrize("shape", [(301, 256, 8, 320), (257, 512, 64, 640), (300, 768, 8, 256), (64, 64, 8, 48)],
                         ids=lambda s: "x".join(map(str, s)))
def test_layer_forward_ws_takes_either_form_with_the_same_bits(gk, shape):
    """grkan_layer_forward_ws (the unfused form beyond 256 output columns, else the fused one)
    gives grkan_layer_forward's bits, and the oracle's values."""
    rows, d_in, n_g, d_out = shape
    inp = inputs(rows, d_in, n_g, d_out, 6100 + rows)
    x, W = bf(inp["x"]), bf(inp["W"])
    A, B = torch.from_numpy(inp["A"]).to(DEV), torch.from_numpy(inp["B"]).to(DEV)
    need = gk.grkan_layer_forward_workspace_size(rows, d_in, d_out, n_g)
    assert (need > 0) == (d_out > 256)
    z = gk.grkan_layer_forward(x, A, B, W, n_g)
    z2 = gk.grkan_layer_forward_ws(x, A, B, W, n_g)
    torch.cuda.synchronize()
    assert torch.equal(z.view(torch.int16), z2.view(torch.int16))
    parity.check_layer(f"layer_ws {shape}", host(z2), layer.forward(inp["x"], inp["A"], inp["B"], inp["W"], n_g),
                       d_in)


@pytest.mark.parametrize("shape", [(301, 256, 272), (300, 3072, 768), (64, 64, 33)],
                         ids=lambda s: "x".join(map(str, s)))
def test_linear_parity(gk, shape):
    rows, d_in, d_out = shape
    log(f"[linear] rows={rows} d_in={d_in} d_out={d_out}")
    inp = inputs(rows, d_in, 8, d_out, 6100 + rows)
    z = gk.grkan_linear_forward(bf(inp["x"]), bf(inp["W"]))
    torch.cuda.synchronize()
    yv = orc.to_f64(inp["x"], "bf16")
    wv = orc.to_f64(inp["W"], "bf16")
    ref = {"z": yv @ wv.T, "amb": np.zeros((rows, d_out)), "mag": np.abs(yv) @ np.abs(wv).T}
    parity.check_layer(f"linear {shape}", host(z), ref, d_in)


def test_linear_output_not_16_byte_aligned(gk):
    """z two bytes past a 16-byte boundary: the kernel must store one bf16 at a time (the
    16-byte row stores need aligned rows) and leave the element before z untouched."""
    rows, d_in, d_out = 300, 256, 272
    log(f"[linear misaligned z] rows={rows} d_in={d_in} d_out={d_out}")
    inp = inputs(rows, d_in, 8, d_out, 6150)
    buf = torch.full((rows * d_out + 8,), 7.0, dtype=torch.bfloat16, device=DEV)
    z = buf[1:1 + rows * d_out].view(rows, d_out)
    gk.grkan_linear_forward(bf(inp["x"]), bf(inp["W"]), out=z)
    torch.cuda.synchronize()
    assert float(buf[0]) == 7.0 and float(buf[-1]) == 7.0
    yv = orc.to_f64(inp["x"], "bf16")
    wv = orc.to_f64(inp["W"], "bf16")
    ref = {"z": yv @ wv.T, "amb": np.zeros((rows, d_out)), "mag": np.abs(yv) @ np.abs(wv).T}
    parity.check_layer("linear misaligned z", host(z), ref, d_in)


def test_layer_special_values(gk):
    """Identity numerators with b = 0 (F = x, so z = x W^T exactly up to accumulation), exact
    zeros, a group at a root of Q, and an identity weight (z = bf16(F(x)))."""
    rows, d_in, n_g = 96, 128, 8
    inp = inputs(rows, d_in, n_g, d_in, 6200)
    inp["x"][::4, :] = 0
    inp["A"][1] = [0, 1, 0, 0, 0, 0]
    inp["B"][1] = 0
    inp["B"][2] = [-0.75, 1.0, 0.0, 0.0]
    inp["x"][1::4, 32:48] = synth.bf16_bits(np.float32([0.75]))[0]
    inp["W"] = synth.bf16_bits(np.eye(d_in, dtype=np.float32))
    x, W = bf(inp["x"]), bf(inp["W"])
    A, B = torch.from_numpy(inp["A"]).to(DEV), torch.from_numpy(inp["B"]).to(DEV)
    z = gk.grkan_layer_forward(x, A, B, W, n_g)
    y = gk.grkan_forward(x, A, B, n_g)
    torch.cuda.synchronize()
    ref = layer.forward(inp["x"], inp["A"], inp["B"], inp["W"], n_g)
    parity.check_layer("layer special", host(z), ref, d_in)
    # identity weight: z is the activation's own bf16 output
    assert torch.equal(z.view(torch.int16), y.view(torch.int16))


def test_layer_empty(gk):
    inp = inputs(4, 64, 8, 16, 6300)
    x = bf(inp["x"])[:0]
    A, B = torch.from_numpy(inp["A"]).to(DEV), torch.from_numpy(inp["B"]).to(DEV)
    z = gk.grkan_layer_forward(x, A, B, bf(inp["W"]), 8)
    assert z.shape == (0, 16)


def test_layer_rejects_unsupported(gk):
    inp = inputs(4, 96, 8, 16, 6400)
    A, B = torch.from_numpy(inp["A"]).to(DEV), torch.from_numpy(inp["B"]).to(DEV)
    with pytest.raises(gk.GRKANError) as e:
        gk.grkan_layer_forward(bf(inp["x"]), A, B, bf(inp["W"]), 8)   # d_in = 96
    assert e.value.status == gk.GRKAN_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", list(synth.LAYER_WORKLOADS))
def test_layer_full_size_sampled(gk, name):
    """The KAT-B MLP layers at full size, in the benchmark's launch configuration: 48 sampled
    rows (first, last, and spread over every row tile) against the oracle."""
    w = synth.WORKLOADS[name]
    log(f"[layer_full] {name}")
    inp = synth.make_inputs(w, need_dy=False)
    x, W = bf(inp["x"]), bf(inp["W"])
    A, B = torch.from_numpy(inp["A"]).to(DEV), torch.from_numpy(inp["B"]).to(DEV)
    z = gk.grkan_layer_forward(x, A, B, W, w.n_groups)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, w.rows - 1], rng.integers(0, w.rows, 46)]))
    zs = host(z[torch.from_numpy(rows).to(DEV)])
    ref = layer.forward(inp["x"][rows], inp["A"], inp["B"], inp["W"], w.n_groups)
    parity.check_layer(f"{name} sampled rows", zs, ref, w.d)


# ---------------------------------------------------------------- backward

def backward_inputs(rows, d_in, n_g, d_out, seed):
    w = synth.custom("layer-bwd", rows, d_in, n_g, io="bf16", seed=seed, d_out=d_out)
    return synth.make_inputs(w)


def check_backward(name, got, ref, sampled_rows=None):
    dx, dA, dB, dW = got
    parity.check_elem_extra(f"{name} dx", host(dx), ref["dx"], ref["dxmag"], ref["dx_amb"], "bf16")
    parity.check_sums(f"{name} dA", dA.cpu().numpy(), ref["dA"], ref["nA"], extra=ref["dA_amb"])
    parity.check_sums(f"{name} dB", dB.cpu().numpy(), ref["dB"], ref["nB"], extra=ref["dB_amb"])
    parity.check_sums(f"{name} dW", dW.cpu().numpy(), ref["dW"], ref["dW_norm"], extra=ref["dW_amb"])


# (rows, d_in, n_groups, d_out): several 256 x 256 tiles, ragged rows and columns, row splits
BWD_SHAPES = [(301, 256, 8, 320), (700, 768, 8, 256), (257, 512, 64, 640), (64, 128, 16, 64), (1, 64, 8, 64),
              (3000, 256, 8, 256)]


@pytest.mark.parametrize("shape", BWD_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_layer_backward_parity(gk, shape):
    rows, d_in, n_g, d_out = shape
    log(f"[layer_bwd] rows={rows} d_in={d_in} n_g={n_g} d_out={d_out}")
    inp = backward_inputs(rows, d_in, n_g, d_out, 7000 + rows)
    x, dz, W = bf(inp["x"]), bf(inp["dz"]), bf(inp["W"])
    A, B = torch.from_numpy(inp["A"]).to(DEV), torch.from_numpy(inp["B"]).to(DEV)
    got = gk.grkan_layer_backward(x, dz, A, B, W, n_g)
    torch.cuda.synchronize()
    ref = layer.backward(inp["x"], inp["dz"], inp["A"], inp["B"], inp["W"], n_g)
    check_backward(f"layer bwd {shape}", got, ref)
    # bitwise reproducible, and dx may be x itself
    got2 = gk.grkan_layer_backward(x, dz, A, B, W, n_g)
    xc = x.clone()
    got3 = gk.grkan_layer_backward(xc, dz, A, B, W, n_g, dx=xc)
    torch.cuda.synchronize()
    for a, b, c in zip(got, got2, got3):
        it = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a.view(it), b.view(it)) and torch.equal(a.view(it), c.view(it))


def test_layer_backward_zero_denominator_groups(gk):
    """Groups with b = 0 (KAT initialises its first GR-KAN layer to the identity, a = (0, 1, 0, ...)
    and b = 0) take the activation backward's D = 1 branch, which also forms the dW operand
    F(x) = P(x) there; the other groups are random.  Both tile variants in one call, against the
    oracle; the identity groups' dB is exactly zero."""
    rows, d_in, n_g, d_out = 700, 512, 8, 256
    log(f"[layer_bwd_b0] rows={rows} d_in={d_in} n_g={n_g} d_out={d_out}")
    inp = backward_inputs(rows, d_in, n_g, d_out, 7300)
    A0, B0 = inp["A"].copy(), inp["B"].copy()
    A0[0] = [0, 1, 0, 0, 0, 0]
    B0[0] = 0
    B0[1] = 0
    B0[5] = -0.0
    x, dz, W = bf(inp["x"]), bf(inp["dz"]), bf(inp["W"])
    A, B = torch.from_numpy(A0).to(DEV), torch.from_numpy(B0).to(DEV)
    got = gk.grkan_layer_backward(x, dz, A, B, W, n_g)
    torch.cuda.synchronize()
    ref = layer.backward(inp["x"], inp["dz"], A0, B0, inp["W"], n_g)
    check_backward("layer bwd b = 0 groups", got, ref)
    dB = got[2].cpu().numpy()
    assert np.all(dB[[0, 1, 5]] == 0)


def test_layer_backward_empty(gk):
    inp = backward_inputs(4, 64, 8, 64, 7100)
    A, B = torch.from_numpy(inp["A"]).to(DEV), torch.from_numpy(inp["B"]).to(DEV)
    dA = torch.full((8, 6), 5.0, device=DEV)
    dB = torch.full((8, 4), 5.0, device=DEV)
    dW = torch.full((64, 64), 5.0, device=DEV)
    gk.grkan_layer_backward(bf(inp["x"])[:0], bf(inp["dz"])[:0], A, B, bf(inp["W"]), 8, dA=dA, dB=dB, dW=dW)
    torch.cuda.synchronize()
    assert not dA.any() and not dB.any() and not dW.any()


@pytest.mark.parametrize("name", list(synth.LAYER_WORKLOADS))
def test_layer_backward_full_size(gk, name):
    """The KAT-B MLP layers' backward at full size, in the benchmark's configuration: dx on
    sampled rows and dW on sampled entries against the oracle one by one; dA, dB against the
    oracle's group sums over every element, on dY from the same matrix kernel (copied back),
    under the literal rule; and within that rule of the activation's own backward
    (grkan_backward) on that dY, which sums the same terms in 4-pass instead of 2-pass tiles."""
    w = synth.WORKLOADS[name]
    log(f"[layer_bwd_full] {name}")
    inp = synth.make_inputs(w)
    x, dz, W = bf(inp["x"]), bf(inp["dz"]), bf(inp["W"])
    A, B = torch.from_numpy(inp["A"]).to(DEV), torch.from_numpy(inp["B"]).to(DEV)
    dx, dA, dB, dW = gk.grkan_layer_backward(x, dz, A, B, W, w.n_groups)
    dy = gk.grkan_linear_forward(dz, W.t().contiguous())
    _, dA2, dB2 = gk.grkan_backward(x, dy, A, B, w.n_groups)
    torch.cuda.synchronize()
    dyh = dy.view(torch.int16).cpu().numpy().view(np.uint16)
    sums = orc.run(inp["x"], inp["A"], inp["B"], w.n_groups, dy=dyh, io="bf16", elements=False)
    del dyh
    for lbl, got, ref, nrm in (("dA", dA, sums["dA"], sums["nA"]), ("dB", dB, sums["dB"], sums["nB"]),
                               ("dA (grkan_backward)", dA2, sums["dA"], sums["nA"]),
                               ("dB (grkan_backward)", dB2, sums["dB"], sums["nB"])):
        parity.check_sums(f"{name} {lbl}", got.cpu().numpy(), ref, nrm, literal=True)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, w.rows - 1], rng.integers(0, w.rows, 30)]))
    ref = layer.backward(inp["x"][rows], inp["dz"][rows], inp["A"], inp["B"], inp["W"], w.n_groups)
    parity.check_elem_extra(f"{name} dx rows", host(dx[torch.from_numpy(rows).to(DEV)]), ref["dx"],
                            ref["dxmag"], ref["dx_amb"], "bf16")
    # dW on 24 sampled entries: column c of bf16(F(x)) over all rows, dotted with column o of dz
    d_g = w.d // w.n_groups
    dzv = orc.to_f64(inp["dz"], "bf16")
    dWh = dW.cpu().numpy()
    for o, c in zip(rng.integers(0, w.d_out, 24), rng.integers(0, w.d, 24)):
        idx = np.arange(w.rows, dtype=np.int64) * w.d + c
        rec = orc.points(inp["x"], inp["A"], inp["B"], w.n_groups, idx, io="bf16")
        f = rec[:, orc.F]
        err = 16.0 * 2.0 ** -24 * rec[:, orc.FMAG]
        fb = layer.bf16_round(f)
        lo, hi = layer.bf16_round(f - err), layer.bf16_round(f + err)
        terms = dzv[:, o] * fb
        refv = math.fsum(terms)
        amb = float(np.sum(np.abs(dzv[:, o]) * np.where(lo != hi, hi - lo, 0.0)))
        norm = float(np.sqrt(np.sum(terms * terms)))
        parity.check_sums(f"{name} dW[{o},{c}]", np.array([dWh[o, c]]), np.array([refv]), np.array([norm]),
                          extra=np.array([amb]))
