"""grkan_backward_noalloc (the backward that allocates nothing: its partial sums live in a
fixed device array of the library) against grkan_backward, the entry point whose scheme it
shares, through the C ABI: bit for bit, on two calls in a row, the second with a smaller input
(the array keeps the first call's contents), and against the fp64 oracle."""
import sys

import numpy as np
import pytest
import torch

from gr_kan_rational_amd import synth
from oracle import oracle as orc
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


def dev_inputs(inp):
    w = inp["workload"]
    if w.io == "bf16":
        cv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)  # noqa: E731
    else:
        cv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    return cv(inp["x"]), cv(inp["dy"]), torch.from_numpy(inp["A"]).to(DEV), torch.from_numpy(inp["B"]).to(DEV)


def bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


# (workload, rows): first a large call, then a smaller one of another shape and dtype.  The first
# sequence's bf16 shape has 16-row tiles like KAT-B hidden and more rows, so that its merge runs in
# chunks (18,752 slots per coefficient, three chunks of 8,192).
CHUNKED = synth.custom("noalloc-chunked-bf16", 300000, 768, 2, io="bf16", seed=960)
SEQUENCES = [
    [(CHUNKED, None), ("kat-b", 1001)],                # 1.5 MB of partial sums and chunk sums, then 20 KB
    [("kat-b-hid-bf16", 201728), ("kat-t", 4097)],     # 4.0 MB (one merge launch of 16 slots per thread),
                                                       # then one of 8
    [("kat-s-hid", 201728), ("tiny", 16)],             # 4.0 MB, then a single tile
    [("kat-b", 201728), ("kat-b-hid-bf16", 1000)],     # 2.0 MB, then a few bf16 tiles
]


def _name(n):
    return n if isinstance(n, str) else n.name


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "-".join(f"{_name(n)}x{r}" for n, r in s))
def test_noalloc_matches_backward_bitwise_on_two_calls(gk, seq):
    for spec, rows in seq:
        inp = synth.make_inputs(spec, rows=rows)
        w = inp["workload"]
        name = w.name
        io = gk.GRKAN_BF16 if w.io == "bf16" else gk.GRKAN_F32
        need = gk.grkan_backward_workspace_size(w.rows, w.d, w.n_groups, io)
        log(f"[noalloc] {name} rows={w.rows} io={w.io}: partial sums {need} B")
        assert 0 < need <= gk.GRKAN_NOALLOC_SCRATCH_BYTES
        x, dy, A, B = dev_inputs(inp)
        dx0, dA0, dB0 = gk.grkan_backward(x, dy, A, B, w.n_groups)
        dx1, dA1, dB1 = gk.grkan_backward_noalloc(x, dy, A, B, w.n_groups)
        torch.cuda.synchronize()
        for a, b in ((dx0, dx1), (dA0, dA1), (dB0, dB1)):
            assert torch.equal(bits(a), bits(b)), name
        if w.rows <= 5000:
            ref = orc.run(inp["x"], inp["A"], inp["B"], w.n_groups, dy=inp["dy"], io=w.io)
            host = dx1.float().cpu().numpy() if w.io == "bf16" else dx1.cpu().numpy()
            parity.check_elem(f"noalloc {name} dX", host, ref["dx"], ref["dxmag"], w.io)
            parity.check_sums(f"noalloc {name} dA", dA1.cpu().numpy(), ref["dA"], ref["nA"], literal=True)
            parity.check_sums(f"noalloc {name} dB", dB1.cpu().numpy(), ref["dB"], ref["nB"], literal=True)
        del x, dy, dx0, dx1


def test_noalloc_rejects_shapes_beyond_its_scratch(gk):
    rows = 5 * 201728  # bf16 KAT-B hidden at five times the batch: > 16 MiB of partial sums
    assert gk.grkan_backward_workspace_size(rows, 3072, 8, gk.GRKAN_BF16) > gk.GRKAN_NOALLOC_SCRATCH_BYTES
    x = torch.empty((16, 3072), dtype=torch.bfloat16, device=DEV)  # never read: rejected first
    A = torch.zeros((8, 6), device=DEV)
    B = torch.zeros((8, 4), device=DEV)
    lib = gk.load_library()
    import ctypes

    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    dA = torch.zeros((8, 6), device=DEV)
    dB = torch.zeros((8, 4), device=DEV)
    st = lib.grkan_backward_noalloc(p(x), p(x), p(A), p(B), p(x), p(dA), p(dB), rows, 3072, 8, gk.GRKAN_BF16,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == gk.GRKAN_ERR_UNSUPPORTED


def test_noalloc_empty_input_writes_zeros(gk):
    x = torch.empty((0, 768), device=DEV)
    A = torch.randn(8, 6, device=DEV)
    B = torch.randn(8, 4, device=DEV)
    dA = torch.full((8, 6), float("nan"), device=DEV)
    dB = torch.full((8, 4), float("nan"), device=DEV)
    gk.grkan_backward_noalloc(x, x, A, B, 8, dA=dA, dB=dB)
    torch.cuda.synchronize()
    assert torch.all(dA == 0) and torch.all(dB == 0)
