"""Pins of the layer oracle (oracle/layer.py) to things other than itself:
torch's float32 -> bfloat16 conversion (round to nearest even), brute-force
sums over the already pinned activation oracle, identity and scaling closed
forms, group locality, and the ambiguity allowance at exact bf16 midpoints.
"""
import math

import numpy as np
import pytest
import torch

from gr_kan_rational_amd import synth
from oracle import layer
from oracle import oracle as orc


def torch_bf16(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),    # bf16 subnormal range
        (rng.standard_normal(20000) * 1e-44).astype(np.float32),    # below it: rounds to 0
    ])
    assert np.array_equal(layer.bf16_round(v.astype(np.float64)), torch_bf16(v))


def test_bf16_round_ties_to_even():
    # midpoints between bf16 neighbours (exact in fp32): 1 + k 2^-7 + 2^-8
    k = np.arange(0, 128)
    mid = (1.0 + k * 2.0 ** -7 + 2.0 ** -8).astype(np.float32)
    got = layer.bf16_round(mid.astype(np.float64))
    assert np.array_equal(got, torch_bf16(mid))
    assert np.all(np.mod(np.round((got - 1.0) * 2 ** 7), 2) == 0)   # the even neighbour


def small_case(rows=3, d_in=16, n_g=2, d_out=5, seed=21):
    w = synth.custom("layer-pin", rows, d_in, n_g, io="bf16", seed=seed, d_out=d_out)
    return synth.make_inputs(w, need_dy=False)


def test_forward_brute_force():
    inp = small_case()
    x, A, B, W = inp["x"], inp["A"], inp["B"], inp["W"]
    rows, d_in = x.shape
    d_out = W.shape[0]
    d_g = d_in // 2
    res = layer.forward(x, A, B, W, 2)
    xv = orc.to_f64(x, "bf16")
    wv = orc.to_f64(W, "bf16")
    for r in range(rows):
        fb = []
        for c in range(d_in):
            g = c // d_g
            f = orc.point(xv[r, c], 0.0, A[g], B[g])[orc.F]
            fb.append(float(torch.tensor(f, dtype=torch.float64).to(torch.bfloat16).double()))
        for o in range(d_out):
            ref = math.fsum(fb[c] * wv[o, c] for c in range(d_in))
            assert abs(res["z"][r, o] - ref) <= 1e-12 * (abs(ref) + 1e-30) + 1e-15
            mag = math.fsum(abs(fb[c] * wv[o, c]) for c in range(d_in))
            assert abs(res["mag"][r, o] - mag) <= 1e-12 * mag


def test_identity_weight_gives_the_rounded_activation():
    inp = small_case(rows=4, d_in=16, d_out=16)
    eye = synth.bf16_bits(np.eye(16, dtype=np.float32))
    res = layer.forward(inp["x"], inp["A"], inp["B"], eye, 2)
    y = orc.run(inp["x"], inp["A"], inp["B"], 2, io="bf16")["y"]
    assert np.array_equal(res["z"], layer.bf16_round(y))


def test_scaling_the_weight_scales_z_exactly():
    inp = small_case(seed=22)
    W2 = synth.bf16_bits(orc.to_f64(inp["W"], "bf16").astype(np.float32) * np.float32(4.0))
    z1 = layer.forward(inp["x"], inp["A"], inp["B"], inp["W"], 2)["z"]
    z4 = layer.forward(inp["x"], inp["A"], inp["B"], W2, 2)["z"]
    assert np.array_equal(z4, 4.0 * z1)


def test_group_locality():
    inp = small_case(rows=5, d_in=32, n_g=4, d_out=6, seed=23)
    W = orc.to_f64(inp["W"], "bf16").astype(np.float32)
    W[:, :16] = 0
    W[:, 24:] = 0                       # only group 2 (channels 16..23) feeds z
    Wb = synth.bf16_bits(W)
    z = layer.forward(inp["x"], inp["A"], inp["B"], Wb, 4)["z"]
    A2, B2 = inp["A"].copy(), inp["B"].copy()
    A2[[0, 1, 3]] += 1.0
    B2[[0, 1, 3]] *= -2.0
    assert np.array_equal(layer.forward(inp["x"], A2, B2, Wb, 4)["z"], z)
    A2[2, 0] += 0.25
    assert not np.array_equal(layer.forward(inp["x"], A2, B2, Wb, 4)["z"], z)


def test_ambiguity_flags_exact_midpoints_only():
    # F = a_0 (b = 0, other a = 0): group 0 sits exactly halfway between two bf16 values,
    # group 1 a quarter step away from that midpoint
    mid = 1.0 + 2.0 ** -8
    A = np.zeros((2, 6), np.float32)
    A[0, 0] = mid
    A[1, 0] = mid + 2.0 ** -10
    B = np.zeros((2, 4), np.float32)
    x = synth.bf16_bits(np.ones((2, 16), np.float32))
    W = synth.bf16_bits(np.ones((3, 16), np.float32))
    res = layer.forward(x, A, B, W, 2)
    fb, width = layer.activation_operand(x, A, B, 2)
    assert np.all(width[:, :8] == 2.0 ** -7) and np.all(width[:, 8:] == 0)
    assert res["n_ambiguous"] == 16
    assert np.allclose(res["amb"], 8 * 2.0 ** -7)
    # either neighbour is within the allowance
    alt = fb.copy()
    alt[:, :8] = 1.0 + 2.0 ** -7          # the other neighbour of the midpoint
    z_alt = alt @ orc.to_f64(W, "bf16").T
    assert np.all(np.abs(z_alt - res["z"]) <= res["amb"])


# ---------------------------------------------------------------- backward

def small_bwd(rows=3, d_in=16, n_g=2, d_out=4, seed=31):
    w = synth.custom("layer-bwd-pin", rows, d_in, n_g, io="bf16", seed=seed, d_out=d_out)
    return synth.make_inputs(w)


def test_backward_brute_force():
    inp = small_bwd()
    x, dz, A, B, W = inp["x"], inp["dz"], inp["A"], inp["B"], inp["W"]
    rows, d_in = x.shape
    d_out = W.shape[0]
    d_g = d_in // 2
    res = layer.backward(x, dz, A, B, W, 2)
    xv, dzv, wv = orc.to_f64(x, "bf16"), orc.to_f64(dz, "bf16"), orc.to_f64(W, "bf16")
    dA = np.zeros((2, 6))
    dB = np.zeros((2, 4))
    for r in range(rows):
        for c in range(d_in):
            g = c // d_g
            dy = float(layer.bf16_round(np.float64(math.fsum(dzv[r, o] * wv[o, c] for o in range(d_out)))))
            rec = orc.point(xv[r, c], dy, A[g], B[g])
            assert abs(res["dx"][r, c] - rec[orc.DX]) <= 1e-13 * (abs(rec[orc.DX]) + 1e-30)
            dA[g] += rec[orc.TA:orc.TA + 6]
            dB[g] += rec[orc.TB:orc.TB + 4]
    assert np.allclose(res["dA"], dA, rtol=1e-12, atol=1e-15)
    assert np.allclose(res["dB"], dB, rtol=1e-12, atol=1e-15)
    for o in range(d_out):
        for c in range(d_in):
            g = c // d_g
            ref = math.fsum(dzv[r, o] * layer.bf16_round(np.float64(orc.point(xv[r, c], 0.0, A[g], B[g])[orc.F]))
                            for r in range(rows))
            assert abs(res["dW"][o, c] - ref) <= 1e-12 * (abs(ref) + 1e-30) + 1e-15


def test_weight_gradient_is_the_derivative_of_the_loss():
    # L(W) = sum dz * z(W) is linear in W: doubling W[o, c] changes L by W[o, c] dW[o, c]
    inp = small_bwd(rows=5, d_in=32, n_g=4, d_out=6, seed=32)
    x, dz, A, B, W = inp["x"], inp["dz"], inp["A"], inp["B"], inp["W"]
    dzv = orc.to_f64(dz, "bf16")
    res = layer.backward(x, dz, A, B, W, 4)

    def loss(Wb):
        return math.fsum((dzv * layer.forward(x, A, B, Wb, 4)["z"]).ravel())

    base = loss(W)
    wv = orc.to_f64(W, "bf16")
    for o, c in [(0, 0), (3, 17), (5, 31), (2, 9)]:
        W2 = W.copy()
        W2[o, c] = synth.bf16_bits(np.float32([2.0 * wv[o, c]]))[0]
        dl = loss(W2) - base
        assert abs(dl - wv[o, c] * res["dW"][o, c]) <= 1e-10 * (abs(dl) + 1e-12)


def test_upstream_ambiguity_at_a_midpoint():
    # dy = 1 * 1 + 2^-8 * 1 = 1 + 2^-8: exactly halfway between bf16 1 and 1 + 2^-7
    dz = synth.bf16_bits(np.float32([[1.0, 2.0 ** -8]]))
    W = synth.bf16_bits(np.ones((2, 8), np.float32))
    dyb, width = layer.upstream(dz, W)
    assert np.all(dyb == 1.0) and np.all(width == 2.0 ** -7)
    A = np.tile(np.float32([0.1, 0.9, -0.2, 0.05, 0.01, -0.02]), (1, 1))
    B = np.tile(np.float32([0.3, -0.1, 0.2, 0.05]), (1, 1))
    x = synth.bf16_bits(np.float32([[0.5, -1.25, 2.0, 0.75, -0.375, 1.5, -2.5, 0.25]]))
    res = layer.backward(x, dz, A, B, W, 1)
    assert res["n_ambiguous_dy"] == 8
    other = orc.run(x, A, B, 1, dy=layer.bf16_bits(np.full((1, 8), 1.0 + 2.0 ** -7)), io="bf16")
    assert np.all(np.abs(other["dx"] - res["dx"]) <= res["dx_amb"] * (1 + 1e-12))
    assert np.all(np.abs(other["dA"] - res["dA"]) <= res["dA_amb"] * (1 + 1e-12))
    assert np.all(np.abs(other["dB"] - res["dB"]) <= res["dB_amb"] * (1 + 1e-12))
    assert np.all(res["dx_amb"] > 0)
