"""C ABI checks that need no GPU: the library loads, exports every function
include/grkan.h declares, and rejects invalid arguments before any HIP call
(so these calls never touch a device; the pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "grkan.h")
LIB = os.path.join(ROOT, "gr_kan_rational_amd", "libgrkan.so")

OK, INVALID, UNSUPPORTED, HIPERR = 0, 1, 2, 3
F32, BF16 = 0, 1
DEFAULT, DET, BLOCK, NAIVE = 0, 1, 2, 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import __graft_entry__

        __graft_entry__.build()
    import torch  # noqa: F401  (load torch's HIP runtime first, as the binding does)

    from gr_kan_rational_amd import binding

    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"GRKAN_API\s+[\w\s\*]*?\b(grkan_\w+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted([
        "grkan_forward", "grkan_backward", "grkan_backward_workspace_size",
        "grkan_status_string", "grkan_query_launch",
        "grkan_pau_supported", "grkan_pau_forward", "grkan_pau_backward",
        "grkan_pau_backward_workspace_size", "grkan_pau_query_launch",
        "grkan_inflated_forward", "grkan_inflated_backward",
        "grkan_layer_forward", "grkan_linear_forward", "grkan_layer_backward",
        "grkan_layer_backward_workspace_size", "grkan_chebykan_forward", "grkan_chebykan_backward",
        "grkan_chebykan_backward_workspace_size", "grkan_backward_noalloc", "grkan_stream_probe",
        "grkan_layer_forward_ws", "grkan_layer_forward_workspace_size"])


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def header_enum(name):
    m = re.search(rf"\b{name}\s*=\s*([^,/\n]+)", open(HEADER).read())
    assert m, name
    return int(eval(m.group(1).replace("1u", "1")))  # "1u << k" as Python


def test_flag_values_are_pinned():
    """The reduction-scheme bits: deterministic is bit 0 (and flags = 0 means the same), the
    two atomic comparison schemes bits 1 and 2; the binding uses the same values."""
    from gr_kan_rational_amd import binding

    assert header_enum("GRKAN_DETERMINISTIC") == DET == binding.GRKAN_DETERMINISTIC == 1
    assert header_enum("GRKAN_BLOCK_ATOMIC") == BLOCK == binding.GRKAN_BLOCK_ATOMIC == 2
    assert header_enum("GRKAN_NAIVE_ATOMIC") == NAIVE == binding.GRKAN_NAIVE_ATOMIC == 4
    assert header_enum("GRKAN_F32") == F32 and header_enum("GRKAN_BF16") == BF16
    assert header_enum("GRKAN_OK") == OK and header_enum("GRKAN_ERR_INVALID_ARG") == INVALID
    assert header_enum("GRKAN_ERR_UNSUPPORTED") == UNSUPPORTED and header_enum("GRKAN_ERR_HIP") == HIPERR
    assert binding._MODES == {"deterministic": DET, "block_atomic": BLOCK, "naive": NAIVE}


def test_deterministic_flag_is_the_default_scheme(lib):
    """flags = GRKAN_DETERMINISTIC asks for exactly what flags = 0 asks for: the same workspace
    and the same validation; combined with an atomic bit it is rejected."""
    for args in ((201728, 768, 8, F32), (201728, 3072, 8, BF16), (100, 40, 8, F32), (16, 32, 8, F32)):
        assert ws(lib, *args, flags=DET) == ws(lib, *args, flags=DEFAULT) > 0
    for f in (DET | BLOCK, DET | NAIVE, BLOCK | NAIVE, DET | BLOCK | NAIVE, 8, 1 << 31):
        assert ws(lib, 201728, 768, 8, flags=f) == 0
        assert bwd(lib, flags=f) == INVALID
    assert bwd(lib, flags=DET, ws_bytes=100) == INVALID      # deterministic needs its workspace
    assert bwd(lib, flags=DET, ws_ptr=None) == INVALID


def test_status_strings(lib):
    for code, word in ((OK, "OK"), (INVALID, "INVALID"), (UNSUPPORTED, "UNSUPPORTED"), (HIPERR, "HIP")):
        assert word in lib.grkan_status_string(code).decode()
    assert lib.grkan_status_string(99)


def ws(lib, rows, d, n_g, io=F32, flags=DEFAULT):
    return lib.grkan_backward_workspace_size(rows, d, n_g, io, flags)


def test_workspace_size(lib):
    # KAT-B backward: 96 channels x 4 B = 24 vectors per group row; 16 rows x 24 = 384 lanes per
    # pass, 2 passes -> 32-row tiles; ceil(201728 / 32) = 6304 tiles; one fp32 partial per
    # (group, coefficient, tile), slots rounded up to a multiple of 8 tiles.  Above 16384 slots
    # the merge adds them in chunks of 8192 and needs one fp64 chunk sum per (group, coefficient,
    # chunk).
    assert ws(lib, 201728, 768, 8) == 8 * 10 * 6304 * 4
    assert ws(lib, 16, 32, 8) == 8 * 10 * 8 * 4             # tiny: a single tile, 8 slots
    assert ws(lib, 201728, 3072, 8, io=BF16) == 8 * 10 * 12608 * 4  # 4 rows x 4 passes: one merge launch
    assert ws(lib, 300000, 3072, 8, io=BF16) == 8 * 10 * 18752 * 4 + 8 * 10 * 3 * 8  # 18752 slots: 3 chunks
    # small grids (under 4096 workgroups at 2 passes) take 1 pass: 16-row tiles
    assert ws(lib, 1000, 768, 8) == 8 * 10 * 64 * 4         # 63 tiles of 16 rows (the last ragged) -> 64 slots
    assert ws(lib, 1025, 768, 8) == 8 * 10 * 72 * 4         # 65 tiles -> 72 slots
    assert ws(lib, 25216, 192, 8) == 8 * 10 * 400 * 4       # KAT-T: 394 tiles of 64 rows -> 400 slots
    assert ws(lib, 201728, 768, 8, flags=BLOCK) == 0        # atomic modes need none
    assert ws(lib, 201728, 768, 8, flags=NAIVE) == 0
    assert ws(lib, 100, 770, 8) == 0                        # d % n_g != 0: rejected
    # 5-channel groups (20 bytes, not whole 16-byte vectors): one channel per lane, 256-row tiles,
    # 64 channels per column block; a group spans at most 2 blocks
    assert ws(lib, 100, 40, 8) == 8 * 10 * 2 * 8 * 4
    # one function per channel at KAT-B: 788 tiles of 256 rows -> 99 bundles -> 792 slots
    assert ws(lib, 201728, 768, 768) == 768 * 10 * 792 * 4
    assert ws(lib, 0, 768, 8) == 0                          # no rows, no tiles


P = 0x10000  # fake, 16-byte aligned "device" addresses: validation never dereferences them


def fwd(lib, x=P, y=P + 0x100000, A=P + 0x200000, B=P + 0x300000, rows=4, d=64, n_g=8, io=F32):
    return lib.grkan_forward(x, y, A, B, rows, d, n_g, io, None)


def bwd(lib, x=P, dy=P + 0x100000, A=P + 0x200000, B=P + 0x300000, dx=P + 0x400000,
        dA=P + 0x500000, dB=P + 0x600000, rows=4, d=64, n_g=8, io=F32, flags=DEFAULT,
        ws_ptr=P + 0x700000, ws_bytes=1 << 20):
    return lib.grkan_backward(x, dy, A, B, dx, dA, dB, rows, d, n_g, io, flags, ws_ptr, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(A=None), INVALID), (dict(B=None), INVALID), (dict(x=None), INVALID), (dict(y=None), INVALID),
    (dict(rows=-1), INVALID), (dict(d=0), INVALID), (dict(n_g=0), INVALID), (dict(d=66), INVALID),
    (dict(io=7), INVALID),
    (dict(x=P + 4), UNSUPPORTED), (dict(y=P + 0x100008), UNSUPPORTED), (dict(A=P + 0x200002), UNSUPPORTED),
    (dict(d=65536 * 4, n_g=65536), UNSUPPORTED),      # more groups than a grid dimension holds
    (dict(y=P + 16), INVALID),                       # partial overlap of y and x
    (dict(y=P + 0x200000 - 16), INVALID),             # y runs into A
])
def test_forward_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code


def test_forward_empty_is_ok_without_device(lib):
    # rows == 0 is a valid no-op that returns before any HIP call; null data pointers are fine.
    assert fwd(lib, x=None, y=None, rows=0) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(dA=None), INVALID), (dict(dB=None), INVALID), (dict(dx=None), INVALID), (dict(dy=None), INVALID),
    (dict(flags=8), INVALID), (dict(flags=BLOCK | NAIVE), INVALID), (dict(flags=DET | BLOCK), INVALID),
    (dict(ws_ptr=None), INVALID), (dict(ws_bytes=100), INVALID),
    (dict(ws_ptr=P + 0x700008), UNSUPPORTED),
    (dict(dx=P + 16), INVALID),                      # dx partially overlaps x
    (dict(dA=P + 0x600000 + 8), INVALID),            # dA overlaps dB
    (dict(dA=P + 64), INVALID),                      # dA inside x
    (dict(ws_ptr=P + 0x400000 - 64), INVALID),       # workspace runs into dx
    (dict(dy=P + 0x100002), UNSUPPORTED),
    (dict(dB=P + 0x600001), UNSUPPORTED),
])
def test_backward_rejects(lib, kw, code):
    assert bwd(lib, **kw) == code


def test_backward_atomic_mode_needs_no_workspace(lib):
    # Validation passes; the call then needs the device.  Without one the HIP query fails
    # cleanly with GRKAN_ERR_HIP rather than crashing.
    import torch

    if torch.cuda.is_available():
        pytest.skip("only meaningful without a GPU")
    assert bwd(lib, flags=BLOCK, ws_ptr=None, ws_bytes=0) == HIPERR


# ---------------------------------------------------------------- PAU family

PAIRS = [(5, 4), (3, 2), (4, 3), (6, 5), (7, 6), (2, 1), (4, 4), (5, 0)]


def test_pau_supported_pairs(lib):
    for m, n in PAIRS:
        assert lib.grkan_pau_supported(m, n) == 1, (m, n)
    for m, n in ((5, 3), (9, 9), (0, 0), (-1, 4), (8, 7)):
        assert lib.grkan_pau_supported(m, n) == 0, (m, n)


def pws(lib, rows, d, n_g, m, n, io=F32, flags=DEFAULT):
    return lib.grkan_pau_backward_workspace_size(rows, d, n_g, m, n, io, flags)


def test_pau_workspace_size(lib):
    # One fp32 partial per (group, coefficient, part, tile); m + 1 + n coefficients.
    assert pws(lib, 201728, 768, 8, 5, 4) == ws(lib, 201728, 768, 8)
    assert pws(lib, 201728, 768, 8, 3, 2) == 8 * 6 * 6304 * 4     # 2 passes of 16 rows: 32-row tiles
    assert pws(lib, 201728, 768, 8, 7, 6) == 8 * 14 * 12608 * 4     # 16-row tiles: one merge launch
    assert pws(lib, 201728, 768, 8, 5, 0) == 8 * 6 * 6304 * 4     # polynomial: no dB sums
    # n_groups = 1 (one PAU for all channels): a 192-vector segment, two rows per pass, 4-row tiles
    assert pws(lib, 201728, 768, 1, 5, 4) == 1 * 10 * 50432 * 4 + 1 * 10 * 7 * 8
    # a 768-vector segment is cut into 2 parts of 384 vectors (one row per pass, 2-row tiles)
    assert pws(lib, 201728, 3072, 1, 5, 4) == 1 * 10 * 4 * 50432 * 4 + 1 * 10 * 25 * 8
    # 1026 vectors per segment (16416 bytes): 3 parts of 342
    assert pws(lib, 4, 8 * 4104, 8, 5, 4) == 8 * 10 * 3 * 8 * 4
    assert pws(lib, 100, 768, 8, 5, 3) == 0                        # pair not compiled in
    assert pws(lib, 100, 768, 8, 3, 2, flags=BLOCK) == 0


def pfwd(lib, m, n, x=P, y=P + 0x100000, A=P + 0x200000, B=P + 0x300000, rows=4, d=64, n_g=8, io=F32):
    return lib.grkan_pau_forward(x, y, A, B, rows, d, n_g, m, n, io, None)


def pbwd(lib, m, n, x=P, dy=P + 0x100000, A=P + 0x200000, B=P + 0x300000, dx=P + 0x400000,
         dA=P + 0x500000, dB=P + 0x600000, rows=4, d=64, n_g=8, io=F32, flags=DEFAULT,
         ws_ptr=P + 0x700000, ws_bytes=1 << 20):
    return lib.grkan_pau_backward(x, dy, A, B, dx, dA, dB, rows, d, n_g, m, n, io, flags, ws_ptr,
                                  ws_bytes, None)


@pytest.mark.parametrize("m,n,code", [((5), 3, UNSUPPORTED), (9, 9, UNSUPPORTED), (-1, 2, INVALID),
                                      (3, -2, INVALID)])
def test_pau_rejects_degrees(lib, m, n, code):
    assert pfwd(lib, m, n) == code
    assert pbwd(lib, m, n) == code


def test_pau_rejects_before_any_device_call(lib):
    assert pfwd(lib, 3, 2, B=None) == INVALID                      # n > 0 needs B
    assert pbwd(lib, 3, 2, dB=None) == INVALID
    assert pbwd(lib, 3, 2, flags=NAIVE) == UNSUPPORTED             # naive baseline: GR-KAN only
    assert pbwd(lib, 7, 6, dA=P + 0x600000 - 8 * 8 * 4 + 8) == INVALID  # dA [8][8] runs into dB
    # n = 0: B and dB may be NULL; rows == 0 returns before any HIP call
    assert pfwd(lib, 5, 0, x=None, y=None, B=None, rows=0) == OK


# ------------------------------------------------------- FLOP-inflation probe

def ifwd(lib, repeat, x=P, y=P + 0x100000, A=P + 0x200000, B=P + 0x300000, rows=4, d=64, n_g=8, io=F32):
    return lib.grkan_inflated_forward(x, y, A, B, rows, d, n_g, io, repeat, None)


def ibwd(lib, repeat, x=P, dy=P + 0x100000, A=P + 0x200000, B=P + 0x300000, dx=P + 0x400000,
         dA=P + 0x500000, dB=P + 0x600000, rows=4, d=64, n_g=8, io=F32, flags=DEFAULT,
         ws_ptr=P + 0x700000, ws_bytes=1 << 20):
    return lib.grkan_inflated_backward(x, dy, A, B, dx, dA, dB, rows, d, n_g, io, flags, repeat,
                                       ws_ptr, ws_bytes, None)


@pytest.mark.parametrize("repeat", [0, 3, 5, 16, -1])
def test_inflated_rejects_repeat(lib, repeat):
    assert ifwd(lib, repeat) == INVALID
    assert ibwd(lib, repeat) == INVALID


@pytest.mark.parametrize("repeat", [1, 2, 4, 8])
def test_inflated_validates_like_the_plain_calls(lib, repeat):
    assert ifwd(lib, repeat, A=None) == INVALID
    assert ifwd(lib, repeat, y=P + 16) == INVALID
    assert ifwd(lib, repeat, x=P + 4) == UNSUPPORTED
    assert ibwd(lib, repeat, ws_bytes=100) == INVALID
    assert ibwd(lib, repeat, dA=P + 0x600000 + 8) == INVALID
    assert ibwd(lib, repeat, flags=BLOCK | NAIVE) == INVALID
    # rows == 0 returns before any HIP call
    assert ifwd(lib, repeat, x=None, y=None, rows=0) == OK


@pytest.mark.parametrize("repeat", [2, 4, 8])
def test_inflated_limits(lib, repeat):
    # 5-channel fp32 groups (20-byte row segments) take the one-channel-per-lane kernels, which
    # have no inflated variant; nor has the naive per-element-atomic baseline.
    assert ifwd(lib, repeat, d=40) == UNSUPPORTED
    assert ibwd(lib, repeat, d=40) == UNSUPPORTED
    assert ibwd(lib, repeat, flags=NAIVE) == UNSUPPORTED
    # the plain kernels still take those (validation passes on to the device)
    assert fwd(lib, d=40, rows=0, x=None, y=None) == OK


# ------------------------------------------------------------------ the layer

def lfwd(lib, x=P, A=P + 0x200000, B=P + 0x300000, W=P + 0x400000, z=P + 0x800000, rows=4, d_in=256,
         d_out=32, n_g=8):
    return lib.grkan_layer_forward(x, A, B, W, z, rows, d_in, d_out, n_g, None)


def linfwd(lib, y=P, W=P + 0x400000, z=P + 0x800000, rows=4, d_in=256, d_out=32):
    return lib.grkan_linear_forward(y, W, z, rows, d_in, d_out, None)


@pytest.mark.parametrize("kw,code", [
    (dict(A=None), INVALID), (dict(B=None), INVALID), (dict(W=None), INVALID), (dict(x=None), INVALID),
    (dict(z=None), INVALID), (dict(rows=-1), INVALID), (dict(d_in=0), INVALID), (dict(d_out=0), INVALID),
    (dict(n_g=0), INVALID), (dict(n_g=3), INVALID),            # 256 % 3 != 0
    (dict(d_in=96, n_g=8), UNSUPPORTED),                       # d_in not a multiple of 64
    (dict(n_g=64, d_in=256), UNSUPPORTED),                     # 4-channel groups: not a multiple of 8
    (dict(n_g=128, d_in=8192), UNSUPPORTED),                   # more than 64 groups
    (dict(rows=1 << 31), UNSUPPORTED), (dict(d_out=1 << 31), UNSUPPORTED),
    (dict(x=P + 8), UNSUPPORTED), (dict(W=P + 0x400008), UNSUPPORTED), (dict(z=P + 0x800001), UNSUPPORTED),
    (dict(A=P + 0x200002), UNSUPPORTED),
    (dict(z=P + 64), INVALID),                                 # z inside x
    (dict(z=P + 0x400000 - 64), INVALID),                      # z runs into W
])
def test_layer_rejects(lib, kw, code):
    assert lfwd(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(W=None), INVALID), (dict(y=None), INVALID), (dict(z=None), INVALID), (dict(rows=-1), INVALID),
    (dict(d_in=96), UNSUPPORTED), (dict(y=P + 8), UNSUPPORTED), (dict(z=P + 64), INVALID),
])
def test_linear_rejects(lib, kw, code):
    assert linfwd(lib, **kw) == code


def test_layer_empty_is_ok_without_device(lib):
    assert lfwd(lib, x=None, z=None, rows=0) == OK
    assert linfwd(lib, y=None, z=None, rows=0) == OK


def lbwd(lib, x=P, dz=P + 0x100000, A=P + 0x200000, B=P + 0x300000, W=P + 0x400000, dx=P + 0x800000,
         dA=P + 0x900000, dB=P + 0x910000, dW=P + 0xA00000, rows=4, d_in=256, d_out=64, n_g=8,
         ws=P + 0x1000000, ws_bytes=1 << 30):
    return lib.grkan_layer_backward(x, dz, A, B, W, dx, dA, dB, dW, rows, d_in, d_out, n_g, ws, ws_bytes, None)


def test_layer_backward_workspace_size(lib):
    f = lib.grkan_layer_backward_workspace_size
    # KAT-B layer 2: W^T (768 x 3072 bf16), one [rows][3072] bf16 buffer, the bf16 activation
    # backward's partials, 14 row splits of fp32 dW partials (at most 16384 rows each: 13 at
    # least; 36 output tiles x 14 = 504 workgroups fill two rounds of 256 to 98%, 13 would fill
    # 91%), each piece 256-byte aligned.  The activation backward that also stores F runs 2
    # passes per workgroup (8-row tiles: 25,216 slots), not the 4 of grkan_backward: fp32
    # partials [8 groups][10 coefficients][25,216], then 4 fp64 chunk sums (8,192 slots each)
    # per coefficient.
    a256 = lambda v: (v + 255) // 256 * 256
    act = 8 * 10 * 25216 * 4 + 8 * 10 * 4 * 8
    # twice the partials of grkan_backward's 16-row tiles, which one merge launch adds (12,608 slots)
    assert 8 * 10 * 25216 * 4 == 2 * lib.grkan_backward_workspace_size(201728, 3072, 8, BF16, 0)
    assert f(201728, 3072, 768, 8) == (a256(768 * 3072 * 2) + a256(201728 * 3072 * 2) + a256(act)
                                      + a256(14 * 768 * 3072 * 4))
    assert f(0, 256, 64, 8) == 0
    assert f(100, 256, 96, 8) == 0      # d_out not a multiple of 64
    assert f(100, 96, 64, 8) == 0       # d_in not a multiple of 64


@pytest.mark.parametrize("kw,code", [
    (dict(A=None), INVALID), (dict(dW=None), INVALID), (dict(dx=None), INVALID), (dict(dz=None), INVALID),
    (dict(ws=None), INVALID), (dict(ws_bytes=1000), INVALID), (dict(d_out=96), UNSUPPORTED),
    (dict(d_in=96), UNSUPPORTED), (dict(n_g=3), INVALID), (dict(ws=P + 0x1000010), UNSUPPORTED),
    (dict(dx=P + 64), INVALID),                        # dx partly overlaps x
    (dict(dx=P + 0x100000), INVALID),                  # dx overlaps dz
    (dict(dW=P + 0x900000 + 8), INVALID),              # dW overlaps dA
    (dict(ws=P + 0x400000), INVALID),                  # workspace overlaps W
    (dict(dW=P + 0x3), UNSUPPORTED),
])
def test_layer_backward_rejects(lib, kw, code):
    assert lbwd(lib, **kw) == code


# ------------------------------------------------------------ Chebyshev KAN

def cfwd(lib, x=P, C=P + 0x400000, y=P + 0x800000, rows=4, d_in=64, d_out=64, deg=7):
    return lib.grkan_chebykan_forward(x, C, y, rows, d_in, d_out, deg, None)


def cbwd(lib, x=P, dy=P + 0x100000, C=P + 0x400000, dx=P + 0x800000, dC=P + 0xA00000, rows=4, d_in=64,
         d_out=64, deg=7, ws=P + 0x1000000, ws_bytes=1 << 30):
    return lib.grkan_chebykan_backward(x, dy, C, dx, dC, rows, d_in, d_out, deg, ws, ws_bytes, None)


def test_chebykan_workspace_size(lib):
    f = lib.grkan_chebykan_backward_workspace_size
    a256 = lambda v: (v + 255) // 256 * 256
    # KAT-B shape: C^T (6144 x 768 bf16) and the dC split partials: 3 x 24 = 72 output tiles x 14
    # splits = 1008 workgroups (four rounds of 256, 98% full) of fp32 [768][6144]
    assert f(201728, 768, 768, 7) == a256(6144 * 768 * 2) + a256(14 * 768 * 6144 * 4)
    assert f(0, 64, 64, 7) == 0
    assert f(10, 64, 96, 7) == 0        # d_out not a multiple of 64
    assert f(10, 64, 64, 3) == 0        # degree 7 only


@pytest.mark.parametrize("kw,code", [
    (dict(C=None), INVALID), (dict(x=None), INVALID), (dict(y=None), INVALID), (dict(rows=-1), INVALID),
    (dict(deg=3), UNSUPPORTED), (dict(deg=-1), INVALID), (dict(d_in=4), UNSUPPORTED),
    (dict(C=P + 0x400008), UNSUPPORTED), (dict(x=P + 1), UNSUPPORTED), (dict(y=P + 64), INVALID),
])
def test_chebykan_forward_rejects(lib, kw, code):
    assert cfwd(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dC=None), INVALID), (dict(dx=None), INVALID), (dict(ws=None), INVALID), (dict(ws_bytes=100), INVALID),
    (dict(d_out=96), UNSUPPORTED), (dict(x=P + 2), UNSUPPORTED), (dict(dx=P + 64), INVALID),
    (dict(dC=P + 0x400000), INVALID), (dict(ws=P + 0x1000010), UNSUPPORTED), (dict(ws=P + 0x800000), INVALID),
])
def test_chebykan_backward_rejects(lib, kw, code):
    assert cbwd(lib, **kw) == code


def test_chebykan_empty_is_ok_without_device(lib):
    assert cfwd(lib, x=None, y=None, rows=0) == OK


# ------------------------------------------------- backward without allocation

def nbwd(lib, x=P, dy=P + 0x100000, A=P + 0x200000, B=P + 0x300000, dx=P + 0x400000,
         dA=P + 0x500000, dB=P + 0x600000, rows=4, d=64, n_g=8, io=F32):
    return lib.grkan_backward_noalloc(x, dy, A, B, dx, dA, dB, rows, d, n_g, io, None)


def test_noalloc_scratch_limit_is_pinned():
    from gr_kan_rational_amd import binding

    m = re.search(r"#define GRKAN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == binding.GRKAN_NOALLOC_SCRATCH_BYTES == 16 << 20


@pytest.mark.parametrize("kw,code", [
    (dict(dA=None), INVALID), (dict(dx=None), INVALID), (dict(d=66), INVALID), (dict(io=7), INVALID),
    (dict(dx=P + 16), INVALID), (dict(dA=P + 0x600000 + 8), INVALID), (dict(x=P + 4), UNSUPPORTED),
    # bf16 KAT-B hidden at 5x the batch: 20.2 MB of partial sums > the 16 MiB array
    (dict(rows=5 * 201728, d=3072, io=BF16), UNSUPPORTED),
])
def test_noalloc_rejects_before_any_device_call(lib, kw, code):
    assert nbwd(lib, **kw) == code


def test_noalloc_covers_the_gr_kan_workloads(lib):
    """The five GR-KAN workloads fit the array (their partial sums are what the workspace query
    reports), and so does the KAT-B hidden bf16 shape at four times the batch."""
    for rows, d, io in ((16, 32, F32), (25216, 192, F32), (201728, 1536, F32), (201728, 768, F32),
                        (201728, 3072, BF16), (4 * 201728, 3072, BF16)):
        assert 0 < ws(lib, rows, d, 8, io) <= 16 << 20


# ------------------------------------------------------- streaming ceiling probe

@pytest.mark.parametrize("args,code", [
    ((P, P + 0x1000, P + 0x2000, -16), INVALID), ((None, P, P + 0x2000, 64), INVALID),
    ((P, P + 0x1000, P + 0x2000, 24), UNSUPPORTED), ((P + 8, P + 0x1000, P + 0x2000, 64), UNSUPPORTED),
    ((P, P + 0x1000, P + 16, 64), INVALID),      # c partially overlaps a
    ((None, None, None, 0), OK),                 # empty: no HIP call
])
def test_stream_probe_validates_before_any_device_call(lib, args, code):
    assert lib.grkan_stream_probe(*args, None) == code


# ------------------------------------------------------ layer forward with a workspace

def test_layer_forward_workspace_size(lib):
    # the unfused form (one bf16 copy of F(x)) beyond one 256-column tile of z, else none
    assert lib.grkan_layer_forward_workspace_size(201728, 768, 3072, 8) == 201728 * 768 * 2
    assert lib.grkan_layer_forward_workspace_size(201728, 3072, 768, 8) == 201728 * 3072 * 2
    assert lib.grkan_layer_forward_workspace_size(1000, 768, 256, 8) == 0
    assert lib.grkan_layer_forward_workspace_size(0, 768, 3072, 8) == 0
    assert lib.grkan_layer_forward_workspace_size(1000, 100, 3072, 8) == 0   # rejected shape


@pytest.mark.parametrize("kw,code", [
    (dict(ws_bytes=100), INVALID), (dict(ws_ptr=None), INVALID), (dict(ws_ptr=P + 0x700008), UNSUPPORTED),
    (dict(ws_ptr=P + 64), INVALID),                   # workspace overlaps x
    (dict(A=None), INVALID), (dict(z=P + 0x600002 + 1), UNSUPPORTED), (dict(d_in=100), UNSUPPORTED),
])
def test_layer_forward_ws_rejects(lib, kw, code):
    args = dict(x=P, A=P + 0x200000, B=P + 0x300000, W=P + 0x400000, z=P + 0x600000, rows=64, d_in=64,
                d_out=512, n_g=8, ws_ptr=P + 0x700000, ws_bytes=1 << 20)
    args.update(kw)
    assert lib.grkan_layer_forward_ws(args["x"], args["A"], args["B"], args["W"], args["z"], args["rows"],
                                      args["d_in"], args["d_out"], args["n_g"], args["ws_ptr"], args["ws_bytes"],
                                      None) == code
