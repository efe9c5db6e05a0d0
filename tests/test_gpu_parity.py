"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

* reduced sizes: every workload's recipe at a row count that spans several
  row tiles per workgroup plus a ragged tail, compared element by element;
* full sizes (the launch configuration the benchmark times): every element
  of Y and dX, streamed through the oracle in row chunks, sampled edge
  elements once more one by one, and the full group sums;
* special values, exactness invariants, determinism, edge cases.
Tolerances: tests/parity.py.
"""
import os
import sys

import numpy as np
import pytest
import torch

from gr_kan_rational_amd import synth
from oracle import oracle as orc
import fullsize
import parity

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def gk():
    import gr_kan_rational_amd.binding as b

    b.load_library()
    return b


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, io: str) -> torch.Tensor:
    if io == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t: torch.Tensor, io: str) -> np.ndarray:
    """fp32 host copy (bf16 values are exact in fp32)."""
    if io == "bf16":
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def dev_inputs(inp):
    io = inp["workload"].io
    return (to_dev(inp["x"], io), to_dev(inp["dy"], io),
            torch.from_numpy(inp["A"]).to(DEV), torch.from_numpy(inp["B"]).to(DEV))


REDUCED_ROWS = {"tiny": 16, "kat-t": 1000, "kat-s-hid": 301, "kat-b": 1001, "kat-b-hid-bf16": 203}


def atomic_adds(gk, w):
    """fp32 atomic adds per coefficient in GRKAN_BLOCK_ATOMIC mode: one per row tile."""
    io = gk.GRKAN_BF16 if w.io == "bf16" else gk.GRKAN_F32
    return gk.grkan_query_launch(w.rows, w.d, w.n_groups, io, 2)["tiles"]


@pytest.mark.parametrize("name", list(REDUCED_ROWS))
@pytest.mark.parametrize("mode", ["deterministic", "block_atomic"])
def test_parity_reduced(gk, name, mode):
    inp = synth.make_inputs(name, rows=REDUCED_ROWS[name])
    w = inp["workload"]
    log(f"[parity_reduced] {name} rows={w.rows} d={w.d} io={w.io} mode={mode}")
    x, dy, A, B = dev_inputs(inp)
    y = gk.grkan_forward(x, A, B, w.n_groups)
    dx, dA, dB = gk.grkan_backward(x, dy, A, B, w.n_groups, mode=mode)
    torch.cuda.synchronize()
    ref = orc.run(inp["x"], inp["A"], inp["B"], w.n_groups, dy=inp["dy"], io=w.io)
    n_add = atomic_adds(gk, w) if mode == "block_atomic" else 0
    parity.check_elem(f"{name} Y", to_host(y, w.io), ref["y"], ref["ymag"], w.io)
    parity.check_elem(f"{name} dX", to_host(dx, w.io), ref["dx"], ref["dxmag"], w.io)
    # deterministic scheme at GR-KAN's degrees: the literal rule (rel 1e-4, abs 1e-6) is asserted
    det = mode == "deterministic"
    sa = parity.check_sums(f"{name} dA", dA.cpu().numpy(), ref["dA"], ref["nA"], n_add, literal=det)
    sb = parity.check_sums(f"{name} dB", dB.cpu().numpy(), ref["dB"], ref["nB"], n_add, literal=det)
    log(f"[parity_reduced] {name} {mode}: dA {sa} dB {sb}")


def sample_indices(w, n_random=20_000, seed=0):
    """Random flat indices plus the first and last rows and every group boundary of row 0."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, w.elements, size=n_random, dtype=np.int64)
    head = np.arange(0, 2 * w.d, dtype=np.int64)
    tail = np.arange(w.elements - 2 * w.d, w.elements, dtype=np.int64)
    return np.unique(np.concatenate([idx, head, tail]))


def check_points(tag, w, inp, y, dx, idx):
    """The elements at flat indices idx, each evaluated on its own by the oracle."""
    it = torch.from_numpy(idx).to(DEV)
    ys = to_host(y.reshape(-1).index_select(0, it), w.io)
    dxs = to_host(dx.reshape(-1).index_select(0, it), w.io)
    rec = orc.points(inp["x"], inp["A"], inp["B"], w.n_groups, idx, dy=inp["dy"], io=w.io)
    parity.check_elem(f"{tag} Y[points]", ys, rec[:, orc.F], rec[:, orc.FMAG], w.io)
    parity.check_elem(f"{tag} dX[points]", dxs, rec[:, orc.DX], rec[:, orc.DXMAG], w.io)


@pytest.mark.parametrize("name", ["tiny", "kat-t", "kat-s-hid", "kat-b", "kat-b-hid-bf16"])
def test_parity_full_size(gk, name):
    """Full workload shapes in the benchmark's launch configuration: every element of Y and dX,
    and the group sums, in both reduction schemes (the literal dA / dB rule in the
    deterministic one)."""
    w = synth.WORKLOADS[name]
    log(f"[parity_full] {name} shape=({w.batch},{w.seq},{w.d}) io={w.io}: generating inputs")
    inp = synth.make_inputs(w)
    x, dy, A, B = dev_inputs(inp)
    log(f"[parity_full] {name}: forward + backward on GPU")
    y = gk.grkan_forward(x, A, B, w.n_groups)
    dx, dA, dB = gk.grkan_backward(x, dy, A, B, w.n_groups)
    _, dA_at, dB_at = gk.grkan_backward(x, dy, A, B, w.n_groups, mode="block_atomic")
    torch.cuda.synchronize()
    del x, dy
    log(f"[parity_full] {name}: sampled edge elements one by one")
    check_points(name, w, inp, y, dx, sample_indices(w))
    log(f"[parity_full] {name}: every element, streamed through the oracle")
    fullsize.compare_all(f"[parity_full] {name}", w, inp, y, dx, log=log)
    del y, dx
    ref = orc.run(inp["x"], inp["A"], inp["B"], w.n_groups, dy=inp["dy"], io=w.io, elements=False)
    sa = parity.check_sums(f"{name} dA", dA.cpu().numpy(), ref["dA"], ref["nA"], literal=True)
    sb = parity.check_sums(f"{name} dB", dB.cpu().numpy(), ref["dB"], ref["nB"], literal=True)
    n_add = atomic_adds(gk, w)
    ta = parity.check_sums(f"{name} dA block_atomic", dA_at.cpu().numpy(), ref["dA"], ref["nA"], n_add)
    tb = parity.check_sums(f"{name} dB block_atomic", dB_at.cpu().numpy(), ref["dB"], ref["nB"], n_add)
    log(f"[parity_full] {name}: ok dA {sa} dB {sb}; block_atomic dA {ta} dB {tb}")
    golden = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", f"{name}.sums.json")
    if os.path.exists(golden):
        import json

        g = json.load(open(golden))
        np.testing.assert_allclose(np.array(g["dA"]), ref["dA"], rtol=1e-12, atol=0)
        np.testing.assert_allclose(np.array(g["dB"]), ref["dB"], rtol=1e-12, atol=0)


def test_parity_tensors_beyond_4_gib(gk):
    """Tensors of 4.96 GB (fp32 [403456, 3072], twice KAT-B's hidden rows): byte offsets past
    2^31 and 2^32 within one tensor, several launches of whole tile bundles.  Every element
    of Y and dX (and the elements around byte offsets 2^31 and 2^32 once more one by one),
    and the full group sums, against the oracle."""
    w = synth.custom("beyond-4gib", 403456, 3072, 8, io="f32", seed=9100)
    log(f"[parity_4gib] rows={w.rows} d={w.d}: generating inputs")
    inp = synth.make_inputs(w)
    x, dy, A, B = dev_inputs(inp)
    log("[parity_4gib] forward + backward on GPU")
    y = gk.grkan_forward(x, A, B, w.n_groups)
    dx, dA, dB = gk.grkan_backward(x, dy, A, B, w.n_groups)
    torch.cuda.synchronize()
    del x, dy
    edges = np.concatenate([np.arange(e - 3 * w.d, e + 3 * w.d, dtype=np.int64) for e in (1 << 29, 1 << 30)])
    check_points("4gib", w, inp, y, dx, np.unique(np.concatenate([sample_indices(w), edges])))
    log("[parity_4gib] every element, streamed through the oracle")
    fullsize.compare_all("[parity_4gib]", w, inp, y, dx, log=log)
    del y, dx
    ref = orc.run(inp["x"], inp["A"], inp["B"], w.n_groups, dy=inp["dy"], io=w.io, elements=False)
    sa = parity.check_sums("4gib dA", dA.cpu().numpy(), ref["dA"], ref["nA"])
    sb = parity.check_sums("4gib dB", dB.cpu().numpy(), ref["dB"], ref["nB"])
    log(f"[parity_4gib] ok dA {sa} dB {sb}")


def special_inputs():
    """d = 64, 8 groups of 8 channels (32-byte group rows: a second geometry).

    group 0: identity numerator, b = 0          group 1: b = 0, random a
    group 2: Q = x (x - 0.75): exact root 0.75   group 3: Q = x (x^2 - 2): root sqrt 2
    group 4: Q = x (x - 1)^3: values below fp64 resolution next to 1
    groups 5-7: random coefficients.
    x: +-0, fp32 neighbours of the roots, large |x| (8), random."""
    rng = np.random.default_rng(7)
    n_g, d = 8, 64
    A = (rng.standard_normal((n_g, 6)) * 0.5).astype(np.float32)
    B = (rng.standard_normal((n_g, 4)) * 0.5).astype(np.float32)
    A[0] = [0, 1, 0, 0, 0, 0]
    B[0] = 0
    B[1] = 0
    B[2] = [-0.75, 1, 0, 0]
    B[3] = [-2, 0, 1, 0]
    B[4] = [-1, 3, -3, 1]
    rows = 48
    x = rng.standard_normal((rows, d)).astype(np.float32)
    f = np.float32
    one, r2 = f(1), f(np.sqrt(2))
    specials = [f(0), -f(0), f(0.75), np.nextafter(f(0.75), f(0)), np.nextafter(f(0.75), f(1)),
                r2, np.nextafter(r2, f(0)), np.nextafter(r2, f(2)), -r2,
                one, np.nextafter(one, f(0)), np.nextafter(one, f(2)), f(8), f(-8), f(1e-30)]
    for g in range(n_g):
        for i, v in enumerate(specials):
            x[i, g * 8 + i % 8] = v          # special value i of every group
            x[i + 24, g * 8 + (i + 3) % 8] = v  # and again, in another column
    dy = rng.standard_normal((rows, d)).astype(np.float32)
    return x, dy, A, B


def test_special_values(gk):
    x, dy, A, B = special_inputs()
    log("[special] x = +-0, near-root x, b = 0 groups, |x| = 8")
    xt, dyt = torch.from_numpy(x).to(DEV), torch.from_numpy(dy).to(DEV)
    At, Bt = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV)
    y = gk.grkan_forward(xt, At, Bt, 8)
    for mode in ("deterministic", "block_atomic"):
        dx, dA, dB = gk.grkan_backward(xt, dyt, At, Bt, 8, mode=mode)
        ref = orc.run(x, A, B, 8, dy=dy)
        parity.check_elem("special Y", y.cpu().numpy(), ref["y"], ref["ymag"])
        parity.check_elem("special dX", dx.cpu().numpy(), ref["dx"], ref["dxmag"])
        parity.check_sums("special dA", dA.cpu().numpy(), ref["dA"], ref["nA"])
        parity.check_sums("special dB", dB.cpu().numpy(), ref["dB"], ref["nB"])
        # the exact-sign cases: dX at the roots must take s from the exact Q, not from fp32 noise
        assert np.all(dB.cpu().numpy()[:2] == 0)


def test_identity_is_exact(gk):
    """a = x, b = 0 in every group: Y == X and dX == dY bitwise (+0 for -0 allowed)."""
    inp = synth.make_inputs("kat-b", rows=333)
    x, dy, _, _ = dev_inputs(inp)
    A = torch.tensor([[0, 1, 0, 0, 0, 0]] * 8, dtype=torch.float32, device=DEV)
    B = torch.zeros((8, 4), dtype=torch.float32, device=DEV)
    y = gk.grkan_forward(x, A, B, 8)
    dx, dA, dB = gk.grkan_backward(x, dy, A, B, 8)
    assert torch.equal(y, x) and torch.equal(dx, dy)
    assert torch.all(dB == 0)
    A_id = np.tile(np.array([0, 1, 0, 0, 0, 0], np.float32), (8, 1))
    ref = orc.run(inp["x"], A_id, np.zeros((8, 4), np.float32), 8, dy=inp["dy"], elements=False)
    parity.check_sums("identity dA", dA.cpu().numpy(), ref["dA"], ref["nA"], literal=True)


def test_deterministic_mode_is_bitwise_stable_and_linear(gk):
    inp = synth.make_inputs("kat-t", rows=4000)
    x, dy, A, B = dev_inputs(inp)
    r1 = gk.grkan_backward(x, dy, A, B, 8)
    r2 = gk.grkan_backward(x, dy, A, B, 8)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    r3 = gk.grkan_backward(x, 2 * dy, A, B, 8)
    for a, b in zip(r1, r3):
        assert torch.equal(2 * a, b)


def test_groups_do_not_interact(gk):
    """Changing group 5's coefficients leaves every other group's outputs bitwise unchanged."""
    inp = synth.make_inputs("kat-b", rows=257)
    x, dy, A, B = dev_inputs(inp)
    y1 = gk.grkan_forward(x, A, B, 8)
    dx1, dA1, dB1 = gk.grkan_backward(x, dy, A, B, 8)
    A2, B2 = A.clone(), B.clone()
    A2[5] += 0.25
    B2[5] *= -1.5
    y2 = gk.grkan_forward(x, A2, B2, 8)
    dx2, dA2, dB2 = gk.grkan_backward(x, dy, A2, B2, 8)
    keep = torch.ones(768, dtype=torch.bool, device=DEV)
    keep[5 * 96:6 * 96] = False
    assert torch.equal(y1[:, keep], y2[:, keep]) and torch.equal(dx1[:, keep], dx2[:, keep])
    other = [g for g in range(8) if g != 5]
    assert torch.equal(dA1[other], dA2[other]) and torch.equal(dB1[other], dB2[other])
    assert not torch.equal(y1[:, ~keep], y2[:, ~keep])


def test_empty_input(gk):
    x = torch.empty((0, 768), dtype=torch.float32, device=DEV)
    A = torch.randn(8, 6, device=DEV)
    B = torch.randn(8, 4, device=DEV)
    y = gk.grkan_forward(x, A, B, 8)
    assert y.shape == (0, 768)
    for mode in ("deterministic", "block_atomic", "naive"):
        dA = torch.full((8, 6), float("nan"), device=DEV)
        dB = torch.full((8, 4), float("nan"), device=DEV)
        gk.grkan_backward(x, x, A, B, 8, mode=mode, dA=dA, dB=dB)
        assert torch.all(dA == 0) and torch.all(dB == 0)


def test_in_place(gk):
    inp = synth.make_inputs("kat-b", rows=100)
    x, dy, A, B = dev_inputs(inp)
    y = gk.grkan_forward(x, A, B, 8)
    dx, dA, dB = gk.grkan_backward(x, dy, A, B, 8)
    xc, dyc = x.clone(), dy.clone()
    gk.grkan_forward(xc, A, B, 8, out=xc)
    assert torch.equal(xc, y)
    _, dA2, dB2 = gk.grkan_backward(x, dyc, A, B, 8, dx=dyc)
    assert torch.equal(dyc, dx) and torch.equal(dA2, dA) and torch.equal(dB2, dB)


def test_errors_surface_as_exceptions(gk):
    x = torch.randn(10, 769, device=DEV)[:, 1:]  # not contiguous rows
    A = torch.randn(8, 6, device=DEV)
    B = torch.randn(8, 4, device=DEV)
    with pytest.raises(ValueError):
        gk.grkan_forward(x, A, B, 8)
    flat = torch.randn(10 * 768 + 1, device=DEV)[1:].view(10, 768)  # 4-byte misaligned
    with pytest.raises(gk.GRKANError) as e:
        gk.grkan_forward(flat, A, B, 8)
    assert e.value.status == gk.GRKAN_ERR_UNSUPPORTED
    with pytest.raises(gk.GRKANError) as e:
        gk.grkan_forward(torch.randn(4, 42, device=DEV), A, B, 8)  # 42 channels in 8 groups
    assert e.value.status == gk.GRKAN_ERR_INVALID_ARG
    with pytest.raises(gk.GRKANError) as e:
        gk.grkan_backward(torch.randn(4, 768, device=DEV), torch.randn(4, 768, device=DEV), A, B, 8,
                          workspace=torch.empty(8, dtype=torch.uint8, device=DEV))
    assert e.value.status == gk.GRKAN_ERR_INVALID_ARG


def test_binding_refuses_what_the_library_cannot_check(gk):
    """Outputs and workspaces of the wrong size, dtype or device, and host tensors, are refused
    by the binding before any launch (the library sees only their pointers)."""
    x, dy = torch.randn(4, 768, device=DEV), torch.randn(4, 768, device=DEV)
    A, B = torch.randn(8, 6, device=DEV), torch.randn(8, 4, device=DEV)
    for kw in (dict(dA=torch.empty(8, 5, device=DEV)), dict(dB=torch.empty(8, 4, device=DEV).double()),
               dict(dx=torch.empty(4, 767, device=DEV)), dict(workspace=torch.empty(1 << 20, dtype=torch.uint8))):
        with pytest.raises(ValueError):
            gk.grkan_backward(x, dy, A, B, 8, **kw)
    with pytest.raises(ValueError):
        gk.grkan_forward(x, A, B, 8, out=torch.empty(4, 768))
    with pytest.raises(ValueError, match="GPU device"):
        gk.grkan_forward(x.cpu(), A.cpu(), B.cpu(), 8)
    xb = torch.randn(256, 256, device=DEV).bfloat16()
    W = torch.randn(64, 256, device=DEV).bfloat16()
    with pytest.raises(ValueError, match="dW"):
        gk.grkan_layer_backward(xb, torch.randn(256, 64, device=DEV).bfloat16(), A, B, W, 8,
                                dW=torch.empty(64, 256, device=DEV).bfloat16())
    torch.cuda.synchronize()


def test_launch_geometry(gk):
    g = gk.grkan_query_launch(201728, 768, 8, gk.GRKAN_F32, 1)
    log(f"[geometry] KAT-B backward: {g}")
    assert g["block"] % 64 == 0 and g["block"] == g["rows_per_iter"] * 24
    assert g["tiles"] == -(-201728 // (g["rows_per_iter"] * g["unroll"]))
    assert g["grid"] == 8 * 8 * (-(-g["tiles"] // 8))
    assert g["grid"] >= 16 * g["cus"]  # many more workgroups than CUs
    assert g["blocks_per_cu"] >= 1


def test_naive_baseline(gk):
    """The per-element-atomic baseline computes the same dX and, up to its fp32 atomic rounding,
    the same sums."""
    inp = synth.make_inputs("kat-b", rows=401)
    x, dy, A, B = dev_inputs(inp)
    dx_n, dA_n, dB_n = gk.grkan_backward(x, dy, A, B, 8, mode="naive")
    dx, dA, dB = gk.grkan_backward(x, dy, A, B, 8)
    torch.cuda.synchronize()
    ref = orc.run(inp["x"], inp["A"], inp["B"], 8, dy=inp["dy"])
    parity.check_elem("naive dX", dx_n.cpu().numpy(), ref["dx"], ref["dxmag"])
    for got, r, n in ((dA_n, ref["dA"], ref["nA"]), (dB_n, ref["dB"], ref["nB"])):
        err = np.abs(got.cpu().numpy() - r)
        assert np.all(err <= 1e-3 * np.maximum(np.abs(r), n) + 1e-6)


def test_autograd_function(gk):
    inp = synth.make_inputs("kat-t", rows=50)
    x, dy, A, B = dev_inputs(inp)
    xg, Ag, Bg = x.clone().requires_grad_(), A.clone().requires_grad_(), B.clone().requires_grad_()
    y = gk.GRKANFunction.apply(xg, Ag, Bg, 8)
    y.backward(dy)
    dx, dA, dB = gk.grkan_backward(x, dy, A, B, 8)
    assert torch.equal(y.detach(), gk.grkan_forward(x, A, B, 8))
    assert torch.equal(xg.grad, dx) and torch.equal(Ag.grad, dA) and torch.equal(Bg.grad, dB)


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_nan_and_inf_propagate_only_where_they_are(gk, io):
    """Non-finite inputs: NaNs in x (group 3) and in dy (group 6), +-Inf in x (group 1).
    Y is NaN exactly where x is NaN; dX is NaN where x or dy is NaN; both are non-finite at
    +-Inf; the groups holding a NaN or Inf get non-finite dA / dB (NaN for the NaN groups); every
    other element and every other group's dA / dB are bitwise those of the same call on the
    clean inputs (IEEE propagation, nothing leaks across elements or groups)."""
    w = synth.custom("nan-inf", 257, 768, 8, io=io, seed=9200)
    inp = synth.make_inputs(w)
    x, dy, A, B = dev_inputs(inp)
    y0 = gk.grkan_forward(x, A, B, 8)
    dx0, dA0, dB0 = gk.grkan_backward(x, dy, A, B, 8)
    dg = 96
    rng = np.random.default_rng(11)
    xn, dyn = x.clone(), dy.clone()
    nan_x = [(int(r), 3 * dg + int(c)) for r, c in zip(rng.integers(0, 257, 5), rng.integers(0, dg, 5))]
    nan_dy = [(int(r), 6 * dg + int(c)) for r, c in zip(rng.integers(0, 257, 5), rng.integers(0, dg, 5))]
    inf_x = [(0, 1 * dg + 7), (100, 1 * dg + 50), (256, 2 * dg - 1)]
    for r, c in nan_x:
        xn[r, c] = float("nan")
    for r, c in nan_dy:
        dyn[r, c] = float("nan")
    for k, (r, c) in enumerate(inf_x):
        xn[r, c] = float("inf") if k % 2 == 0 else float("-inf")
    log(f"[nan_inf] io={io}: NaN x at {nan_x}, NaN dy at {nan_dy}, Inf x at {inf_x}")
    y = gk.grkan_forward(xn, A, B, 8)
    dx, dA, dB = gk.grkan_backward(xn, dyn, A, B, 8)
    _, dA_at, dB_at = gk.grkan_backward(xn, dyn, A, B, 8, mode="block_atomic")
    torch.cuda.synchronize()
    bad_y = torch.zeros(x.shape, dtype=torch.bool, device=DEV)
    bad_dx = bad_y.clone()
    for r, c in nan_x + inf_x:
        bad_y[r, c] = True
        bad_dx[r, c] = True
    for r, c in nan_dy:
        bad_dx[r, c] = True
    for r, c in nan_x:
        assert torch.isnan(y[r, c]) and torch.isnan(dx[r, c])
    for r, c in nan_dy:
        assert torch.isnan(dx[r, c])
    for r, c in inf_x:
        assert not torch.isfinite(y[r, c]) and not torch.isfinite(dx[r, c])
    assert torch.equal(_bits(y)[~bad_y], _bits(y0)[~bad_y])
    assert torch.equal(_bits(dx)[~bad_dx], _bits(dx0)[~bad_dx])
    for g in (3, 6):
        assert torch.all(torch.isnan(dA[g])) and torch.all(torch.isnan(dB[g]))
        assert torch.all(torch.isnan(dA_at[g])) and torch.all(torch.isnan(dB_at[g]))
    assert not torch.all(torch.isfinite(dA[1])) or not torch.all(torch.isfinite(dB[1]))
    clean = [0, 2, 4, 5, 7]
    assert torch.equal(_bits(dA[clean]), _bits(dA0[clean])) and torch.equal(_bits(dB[clean]), _bits(dB0[clean]))
    assert torch.all(torch.isfinite(dA_at[clean])) and torch.all(torch.isfinite(dB_at[clean]))


def test_flags_zero_and_deterministic_are_the_same_call(gk):
    """flags = 0 and flags = GRKAN_DETERMINISTIC select the same scheme: identical bits."""
    import ctypes

    inp = synth.make_inputs("kat-b", rows=515)
    x, dy, A, B = dev_inputs(inp)
    lib = gk.load_library()
    out = []
    for flags in (0, gk.GRKAN_DETERMINISTIC):
        dx = torch.empty_like(x)
        dA = torch.empty((8, 6), dtype=torch.float32, device=DEV)
        dB = torch.empty((8, 4), dtype=torch.float32, device=DEV)
        n = lib.grkan_backward_workspace_size(515, 768, 8, gk.GRKAN_F32, flags)
        ws = torch.empty(n, dtype=torch.uint8, device=DEV)
        p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        st = lib.grkan_backward(p(x), p(dy), p(A), p(B), p(dx), p(dA), p(dB), 515, 768, 8, gk.GRKAN_F32, flags,
                                p(ws), n, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == gk.GRKAN_OK
        out.append((dx, dA, dB))
    torch.cuda.synchronize()
    for a, b in zip(*out):
        assert torch.equal(_bits(a), _bits(b))


def test_stream_probe_is_the_xor_of_its_inputs(gk):
    """The streaming-ceiling probe the benchmark rates the backward against: c = a XOR b over
    the whole byte range, including a ragged last workgroup, and in place."""
    g = torch.Generator(device="cpu").manual_seed(5)
    for n in (16, 4096 * 4 + 48, 201728 * 768):
        a = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, generator=g).to(DEV)
        b = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, generator=g).to(DEV)
        c = gk.grkan_stream_probe(a, b)
        assert torch.equal(c, a ^ b)
        gk.grkan_stream_probe(a, b, out=a)
        assert torch.equal(a, c)
