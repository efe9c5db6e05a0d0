"""The Python binding's own checks, on the CPU (no device calls).

The binding marshals tensors into the C ABI's plain pointers; the library can
check pointers only for null, alignment and overlap, so the binding refuses
what the library cannot see: host tensors (whose pointers would reach a
kernel), and caller-supplied outputs or workspaces of the wrong dtype, size,
layout or device.  Without the built library every call raises: there is no
other implementation to fall back to.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from gr_kan_rational_amd import binding as gk  # noqa: E402

HAVE_LIB = os.path.exists(gk.LIB_PATH)


def _act(rows=4, d=64, dtype=torch.float32):
    x = torch.zeros(rows, d, dtype=dtype)
    return x, torch.zeros(8, 6), torch.zeros(8, 4)


HOST_CALLS = [
    ("grkan_forward", lambda: gk.grkan_forward(*_act())),
    ("grkan_pau_forward", lambda: gk.grkan_pau_forward(*_act(), 8, 5, 4)),
    ("grkan_inflated_forward", lambda: gk.grkan_inflated_forward(*_act(), 8, 2)),
    ("grkan_backward", lambda: gk.grkan_backward(_act()[0], _act()[0], *_act()[1:])),
    ("grkan_pau_backward", lambda: gk.grkan_pau_backward(_act()[0], _act()[0], *_act()[1:], 8, 5, 4)),
    ("grkan_inflated_backward", lambda: gk.grkan_inflated_backward(_act()[0], _act()[0], *_act()[1:])),
    ("grkan_backward_noalloc", lambda: gk.grkan_backward_noalloc(_act()[0], _act()[0], *_act()[1:])),
    ("grkan_stream_probe", lambda: gk.grkan_stream_probe(torch.zeros(64), torch.zeros(64))),
    ("grkan_layer_forward", lambda: gk.grkan_layer_forward(
        torch.zeros(4, 64, dtype=torch.bfloat16), *_act()[1:], torch.zeros(64, 64, dtype=torch.bfloat16))),
    ("grkan_linear_forward", lambda: gk.grkan_linear_forward(
        torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(64, 64, dtype=torch.bfloat16))),
    ("grkan_layer_backward", lambda: gk.grkan_layer_backward(
        torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(4, 64, dtype=torch.bfloat16), *_act()[1:],
        torch.zeros(64, 64, dtype=torch.bfloat16))),
    ("grkan_chebykan_forward", lambda: gk.grkan_chebykan_forward(
        torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(64, 64, 8, dtype=torch.bfloat16))),
    ("grkan_chebykan_backward", lambda: gk.grkan_chebykan_backward(
        torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(4, 64, dtype=torch.bfloat16),
        torch.zeros(64, 64, 8, dtype=torch.bfloat16))),
]


@pytest.mark.skipif(not HAVE_LIB, reason="libgrkan.so not built")
@pytest.mark.parametrize("name, call", HOST_CALLS, ids=[n for n, _ in HOST_CALLS])
def test_host_tensors_are_refused(name, call):
    with pytest.raises(ValueError, match="GPU device"):
        call()


def test_caller_outputs_are_checked():
    dev = torch.device("cpu")
    gk._check_out(torch.zeros(8, 6), "dA", torch.float32, 48, dev)
    for bad in (torch.zeros(8, 5), torch.zeros(8, 6, dtype=torch.float64), torch.zeros(6, 16)[:, :8].t()):
        with pytest.raises(ValueError, match="dA"):
            gk._check_out(bad, "dA", torch.float32, 48, dev)
    with pytest.raises(ValueError, match="dA"):
        gk._check_out(torch.zeros(8, 6), "dA", torch.float32, 48, torch.device("meta"))


def test_gradient_outputs_are_allocated_or_checked():
    x = torch.zeros(4, 64)
    dx, dA, dB = gk._grad_outputs(x, 8, 5, 4, None, None, None)
    assert dx.shape == x.shape and dA.shape == (8, 6) and dB.shape == (8, 4)
    assert gk._grad_outputs(x, 8, 5, 0, None, None, None)[2] is None
    gk._grad_outputs(x, 8, 5, 4, x, dA, dB)  # in place on x is the library's affair
    for kw in (dict(dx=torch.zeros(4, 32)), dict(dx=torch.zeros(4, 64, dtype=torch.bfloat16)),
               dict(dA=torch.zeros(8, 5)), dict(dB=torch.zeros(8, 6)), dict(dB=torch.zeros(4, 8)[:, :4])):
        args = dict(dx=None, dA=None, dB=None)
        args.update(kw)
        with pytest.raises(ValueError):
            gk._grad_outputs(x, 8, 5, 4, args["dx"], args["dA"], args["dB"])


def test_workspace_size_is_counted_in_bytes():
    dev = torch.device("cpu")
    assert gk._workspace(None, dev) == (None, 0)
    assert gk._workspace(torch.zeros(10, dtype=torch.float32), dev)[1] == 40
    assert gk._workspace(torch.zeros(10, dtype=torch.uint8), dev)[1] == 10
    with pytest.raises(ValueError, match="workspace"):
        gk._workspace(torch.zeros(10, 4)[:, 0], dev)
    with pytest.raises(ValueError, match="workspace"):
        gk._workspace(torch.zeros(10), torch.device("meta"))


def test_missing_library_raises_in_a_fresh_process():
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import torch\n"
            "from gr_kan_rational_amd import binding as gk\n"
            "gk.load_library.__defaults__ = ('/nonexistent/libgrkan.so',)\n"
            "try:\n"
            "    gk.grkan_forward(torch.zeros(4, 64), torch.zeros(8, 6), torch.zeros(8, 4))\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('no error')\n" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert "raised: GR-KAN HIP library not built" in r.stdout, r.stdout
