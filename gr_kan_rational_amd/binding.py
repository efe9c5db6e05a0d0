"""Thin Python binding of libgrkan.so (C ABI in include/grkan.h).

Argument marshalling only: tensors become device pointers, shapes and a
stream handle; every step of the computation runs in the library's HIP
kernels.  The library is loaded on first use; if it is missing or cannot be
loaded, every call raises -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgrkan.so")

GRKAN_OK, GRKAN_ERR_INVALID_ARG, GRKAN_ERR_UNSUPPORTED, GRKAN_ERR_HIP = 0, 1, 2, 3
GRKAN_F32, GRKAN_BF16 = 0, 1
GRKAN_DETERMINISTIC = 1 << 0
GRKAN_BLOCK_ATOMIC = 1 << 1
GRKAN_NAIVE_ATOMIC = 1 << 2
_MODES = {"deterministic": GRKAN_DETERMINISTIC, "block_atomic": GRKAN_BLOCK_ATOMIC,
          "naive": GRKAN_NAIVE_ATOMIC}


class GRKANError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {grkan_status_string(status)}")


class grkan_launch_t(ctypes.Structure):
    _fields_ = [
        ("block", ctypes.c_int32),
        ("rows_per_iter", ctypes.c_int32),
        ("unroll", ctypes.c_int32),
        ("tiles", ctypes.c_int64),
        ("grid", ctypes.c_int64),
        ("cus", ctypes.c_int32),
        ("blocks_per_cu", ctypes.c_int32),
        ("parts", ctypes.c_int32),
        ("part_vecs", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgrkan.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"GR-KAN HIP library not built ({path}); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    vp, i64, i32, u32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    lib.grkan_forward.argtypes = [vp, vp, vp, vp, i64, i64, i32, ctypes.c_int, vp]
    lib.grkan_forward.restype = ctypes.c_int
    lib.grkan_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, ctypes.c_int, u32, vp, sz, vp]
    lib.grkan_backward.restype = ctypes.c_int
    lib.grkan_stream_probe.argtypes = [vp, vp, vp, i64, vp]
    lib.grkan_stream_probe.restype = ctypes.c_int
    lib.grkan_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, ctypes.c_int, vp]
    lib.grkan_backward_noalloc.restype = ctypes.c_int
    lib.grkan_backward_workspace_size.argtypes = [i64, i64, i32, ctypes.c_int, u32]
    lib.grkan_backward_workspace_size.restype = sz
    lib.grkan_status_string.argtypes = [ctypes.c_int]
    lib.grkan_status_string.restype = ctypes.c_char_p
    lib.grkan_query_launch.argtypes = [i64, i64, i32, ctypes.c_int, i32, ctypes.POINTER(grkan_launch_t)]
    lib.grkan_query_launch.restype = ctypes.c_int
    lib.grkan_pau_supported.argtypes = [i32, i32]
    lib.grkan_pau_supported.restype = ctypes.c_int
    lib.grkan_pau_forward.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, ctypes.c_int, vp]
    lib.grkan_pau_forward.restype = ctypes.c_int
    lib.grkan_pau_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, ctypes.c_int,
                                       u32, vp, sz, vp]
    lib.grkan_pau_backward.restype = ctypes.c_int
    lib.grkan_pau_backward_workspace_size.argtypes = [i64, i64, i32, i32, i32, ctypes.c_int, u32]
    lib.grkan_pau_backward_workspace_size.restype = sz
    lib.grkan_pau_query_launch.argtypes = [i64, i64, i32, i32, i32, ctypes.c_int, i32,
                                           ctypes.POINTER(grkan_launch_t)]
    lib.grkan_pau_query_launch.restype = ctypes.c_int
    lib.grkan_inflated_forward.argtypes = [vp, vp, vp, vp, i64, i64, i32, ctypes.c_int, i32, vp]
    lib.grkan_inflated_forward.restype = ctypes.c_int
    lib.grkan_inflated_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, ctypes.c_int, u32,
                                            i32, vp, sz, vp]
    lib.grkan_inflated_backward.restype = ctypes.c_int
    lib.grkan_layer_forward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.grkan_layer_forward.restype = ctypes.c_int
    lib.grkan_layer_forward_ws.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, vp]
    lib.grkan_layer_forward_ws.restype = ctypes.c_int
    lib.grkan_layer_forward_workspace_size.argtypes = [i64, i64, i64, i32]
    lib.grkan_layer_forward_workspace_size.restype = sz
    lib.grkan_linear_forward.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.grkan_linear_forward.restype = ctypes.c_int
    lib.grkan_layer_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, vp]
    lib.grkan_layer_backward.restype = ctypes.c_int
    lib.grkan_layer_backward_workspace_size.argtypes = [i64, i64, i64, i32]
    lib.grkan_layer_backward_workspace_size.restype = sz
    lib.grkan_chebykan_forward.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp]
    lib.grkan_chebykan_forward.restype = ctypes.c_int
    lib.grkan_chebykan_backward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, vp]
    lib.grkan_chebykan_backward.restype = ctypes.c_int
    lib.grkan_chebykan_backward_workspace_size.argtypes = [i64, i64, i64, i32]
    lib.grkan_chebykan_backward_workspace_size.restype = sz
    _lib = lib
    return lib


def grkan_status_string(status: int) -> str:
    return load_library().grkan_status_string(int(status)).decode()


def _io(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GRKAN_F32
    if t.dtype == torch.bfloat16:
        return GRKAN_BF16
    raise TypeError(f"GR-KAN I/O dtype must be float32 or bfloat16, got {t.dtype}")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on_gpu(x: torch.Tensor) -> None:
    # the library computes on the device only: a host tensor's pointer must never reach a kernel
    if x.device.type != "cuda":
        raise ValueError(f"GR-KAN tensors must be on a GPU device, got {x.device}")


def _check_out(t: torch.Tensor, name: str, dtype, numel: int, dev) -> None:
    """A caller-supplied output: the library writes numel elements of dtype through its pointer."""
    if t.dtype != dtype or t.numel() != numel or not t.is_contiguous() or t.device != dev:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of {numel} elements on {dev}")


def _workspace(ws, dev):
    """(pointer, size in bytes) of an optional caller-supplied workspace on dev."""
    if ws is None:
        return None, 0
    if not ws.is_contiguous() or ws.device != dev:
        raise ValueError(f"workspace must be a contiguous tensor on {dev}")
    return _ptr(ws), ws.numel() * ws.element_size()


GRKAN_M, GRKAN_N = 5, 4  # GR-KAN's numerator / denominator degrees


def _check_coefs(A: torch.Tensor, B, n_groups: int, dev, m: int = GRKAN_M, n: int = GRKAN_N) -> None:
    for name, t, k in (("A", A, m + 1), ("B", B, n)):
        if k == 0 and t is None:
            continue
        if t.dtype != torch.float32 or t.device != dev or not t.is_contiguous() or t.numel() != n_groups * k:
            raise ValueError(f"{name} must be a contiguous float32 [{n_groups}, {k}] tensor on {dev}")


def _rows_d(x: torch.Tensor):
    if x.dim() < 1 or not x.is_contiguous():
        raise ValueError("activations must be contiguous with channels last")
    d = x.shape[-1]
    return (x.numel() // d if d else 0), d


def _forward(x, A, B, n_groups, m, n, out, stream, pau, repeat=None):
    lib = load_library()
    io = _io(x)
    _on_gpu(x)
    _check_coefs(A, B, n_groups, x.device, m, n)
    rows, d = _rows_d(x)
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous() or y.device != x.device:
        raise ValueError("out must match x")
    s = ctypes.c_void_p(_stream(stream))
    if repeat is not None:
        name = "grkan_inflated_forward"
        st = lib.grkan_inflated_forward(_ptr(x), _ptr(y), _ptr(A), _ptr(B), rows, d, n_groups, io,
                                        int(repeat), s)
    elif pau:
        name = "grkan_pau_forward"
        st = lib.grkan_pau_forward(_ptr(x), _ptr(y), _ptr(A), _ptr(B), rows, d, n_groups, m, n, io, s)
    else:
        name = "grkan_forward"
        st = lib.grkan_forward(_ptr(x), _ptr(y), _ptr(A), _ptr(B), rows, d, n_groups, io, s)
    if st != GRKAN_OK:
        raise GRKANError(st, name)
    return y


def grkan_forward(x: torch.Tensor, A: torch.Tensor, B: torch.Tensor, n_groups: int = 8,
                  out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = F(x), the group-rational activation, computed by ``grkan_forward``."""
    return _forward(x, A, B, n_groups, GRKAN_M, GRKAN_N, out, stream, pau=False)


def grkan_pau_forward(x: torch.Tensor, A: torch.Tensor, B, n_groups: int, m: int, n: int,
                      out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = F(x) for numerator degree m and denominator degree n (``grkan_pau_forward``);
    A is [n_groups, m+1], B is [n_groups, n] (None when n == 0)."""
    return _forward(x, A, B, n_groups, m, n, out, stream, pau=True)


def grkan_inflated_forward(x: torch.Tensor, A: torch.Tensor, B: torch.Tensor, n_groups: int = 8,
                           repeat: int = 8, out: torch.Tensor | None = None,
                           stream=None) -> torch.Tensor:
    """grkan_forward with each element's rational evaluated `repeat` times
    (``grkan_inflated_forward``, the FLOP-inflation probe): same output, more arithmetic."""
    return _forward(x, A, B, n_groups, GRKAN_M, GRKAN_N, out, stream, pau=False, repeat=repeat)


def grkan_backward_workspace_size(rows: int, d: int, n_groups: int, io: int = GRKAN_F32,
                                  flags: int = 0) -> int:
    return int(load_library().grkan_backward_workspace_size(rows, d, n_groups, io, flags))


def grkan_pau_backward_workspace_size(rows: int, d: int, n_groups: int, m: int, n: int,
                                      io: int = GRKAN_F32, flags: int = 0) -> int:
    return int(load_library().grkan_pau_backward_workspace_size(rows, d, n_groups, m, n, io, flags))


def grkan_pau_supported(m: int, n: int) -> bool:
    return bool(load_library().grkan_pau_supported(m, n))


def _grad_outputs(x, n_groups, m, n, dx, dA, dB):
    """dx, dA [n_groups, m+1], dB [n_groups, n] (None when n == 0): allocated when not given,
    checked when given."""
    if dx is None:
        dx = torch.empty_like(x)
    elif dx.shape != x.shape or dx.dtype != x.dtype or not dx.is_contiguous() or dx.device != x.device:
        raise ValueError("dx must match x")
    if dA is None:
        dA = torch.empty((n_groups, m + 1), dtype=torch.float32, device=x.device)
    _check_out(dA, "dA", torch.float32, n_groups * (m + 1), x.device)
    if n > 0:
        if dB is None:
            dB = torch.empty((n_groups, n), dtype=torch.float32, device=x.device)
        _check_out(dB, "dB", torch.float32, n_groups * n, x.device)
    return dx, dA, dB


def _backward(x, dy, A, B, n_groups, m, n, mode, dx, dA, dB, workspace, stream, pau, repeat=None):
    lib = load_library()
    io = _io(x)
    _on_gpu(x)
    if dy.shape != x.shape or dy.dtype != x.dtype or dy.device != x.device or not dy.is_contiguous():
        raise ValueError("dy must match x")
    _check_coefs(A, B, n_groups, x.device, m, n)
    rows, d = _rows_d(x)
    if mode not in _MODES:
        raise ValueError(f"mode must be one of {sorted(_MODES)}")
    flags = _MODES[mode]
    dx, dA, dB = _grad_outputs(x, n_groups, m, n, dx, dA, dB)
    if pau:
        ws_bytes = lib.grkan_pau_backward_workspace_size(rows, d, n_groups, m, n, io, flags)
    else:
        ws_bytes = lib.grkan_backward_workspace_size(rows, d, n_groups, io, flags)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    wsp, wsn = _workspace(workspace, x.device)
    s = ctypes.c_void_p(_stream(stream))
    if repeat is not None:
        name = "grkan_inflated_backward"
        st = lib.grkan_inflated_backward(_ptr(x), _ptr(dy), _ptr(A), _ptr(B), _ptr(dx), _ptr(dA),
                                         _ptr(dB), rows, d, n_groups, io, flags, int(repeat), wsp, wsn, s)
    elif pau:
        name = "grkan_pau_backward"
        st = lib.grkan_pau_backward(_ptr(x), _ptr(dy), _ptr(A), _ptr(B), _ptr(dx), _ptr(dA), _ptr(dB),
                                    rows, d, n_groups, m, n, io, flags, wsp, wsn, s)
    else:
        name = "grkan_backward"
        st = lib.grkan_backward(_ptr(x), _ptr(dy), _ptr(A), _ptr(B), _ptr(dx), _ptr(dA), _ptr(dB),
                                rows, d, n_groups, io, flags, wsp, wsn, s)
    if st != GRKAN_OK:
        raise GRKANError(st, name)
    return dx, dA, dB


def grkan_backward(x: torch.Tensor, dy: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                   n_groups: int = 8, mode: str = "deterministic",
                   dx: torch.Tensor | None = None, dA: torch.Tensor | None = None,
                   dB: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   stream=None):
    """(dx, dA, dB) of the group-rational activation, computed by ``grkan_backward``.

    ``mode``: "deterministic" (the two-stage fixed-order reduction, default),
    "block_atomic" (one fp32 atomic per coefficient per workgroup) or "naive"
    (ten fp32 atomics per element); the last two are for comparison only.
    """
    return _backward(x, dy, A, B, n_groups, GRKAN_M, GRKAN_N, mode, dx, dA, dB, workspace, stream,
                     pau=False)


def grkan_backward_noalloc(x: torch.Tensor, dy: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                           n_groups: int = 8, dx: torch.Tensor | None = None, dA: torch.Tensor | None = None,
                           dB: torch.Tensor | None = None, stream=None):
    """(dx, dA, dB) by ``grkan_backward_noalloc``: the deterministic scheme with the library's own
    fixed scratch array instead of a workspace (no device allocation inside the call; the output
    tensors are allocated here only when not given)."""
    lib = load_library()
    io = _io(x)
    _on_gpu(x)
    if dy.shape != x.shape or dy.dtype != x.dtype or dy.device != x.device or not dy.is_contiguous():
        raise ValueError("dy must match x")
    _check_coefs(A, B, n_groups, x.device)
    rows, d = _rows_d(x)
    dx, dA, dB = _grad_outputs(x, n_groups, GRKAN_M, GRKAN_N, dx, dA, dB)
    st = lib.grkan_backward_noalloc(_ptr(x), _ptr(dy), _ptr(A), _ptr(B), _ptr(dx), _ptr(dA), _ptr(dB),
                                    rows, d, n_groups, io, ctypes.c_void_p(_stream(stream)))
    if st != GRKAN_OK:
        raise GRKANError(st, "grkan_backward_noalloc")
    return dx, dA, dB


GRKAN_NOALLOC_SCRATCH_BYTES = 16 << 20


def grkan_stream_probe(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """out = a XOR b over the tensors' bytes (``grkan_stream_probe``, the streaming ceiling
    probe: two reads and one write per 16 bytes, as the backward moves)."""
    _on_gpu(a)
    if a.numel() * a.element_size() != b.numel() * b.element_size() or not (a.is_contiguous() and b.is_contiguous()) \
            or b.device != a.device:
        raise ValueError("a and b must be contiguous tensors of the same byte size on one device")
    out = torch.empty_like(a) if out is None else out
    nbytes = a.numel() * a.element_size()
    if out.numel() * out.element_size() != nbytes or not out.is_contiguous() or out.device != a.device:
        raise ValueError("out must be a contiguous tensor of a's byte size on a's device")
    st = load_library().grkan_stream_probe(_ptr(a), _ptr(b), _ptr(out), nbytes, ctypes.c_void_p(_stream(stream)))
    if st != GRKAN_OK:
        raise GRKANError(st, "grkan_stream_probe")
    return out


def grkan_pau_backward(x: torch.Tensor, dy: torch.Tensor, A: torch.Tensor, B, n_groups: int,
                       m: int, n: int, mode: str = "deterministic",
                       dx: torch.Tensor | None = None, dA: torch.Tensor | None = None,
                       dB: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                       stream=None):
    """(dx, dA, dB) for degrees (m, n) (``grkan_pau_backward``); dB is None when n == 0."""
    return _backward(x, dy, A, B, n_groups, m, n, mode, dx, dA, dB, workspace, stream, pau=True)


def grkan_inflated_backward(x: torch.Tensor, dy: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                            n_groups: int = 8, repeat: int = 8, mode: str = "deterministic",
                            dx: torch.Tensor | None = None, dA: torch.Tensor | None = None,
                            dB: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                            stream=None):
    """grkan_backward with each element evaluated `repeat` times
    (``grkan_inflated_backward``, the FLOP-inflation probe): same outputs, more arithmetic."""
    return _backward(x, dy, A, B, n_groups, GRKAN_M, GRKAN_N, mode, dx, dA, dB, workspace, stream,
                     pau=False, repeat=repeat)


def _layer_dims(x, W):
    if x.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise TypeError("the layer takes bfloat16 x and W")
    _on_gpu(x)
    if W.dim() != 2 or not W.is_contiguous() or W.device != x.device:
        raise ValueError("W must be a contiguous [d_out, d_in] tensor on x's device")
    rows, d_in = _rows_d(x)
    if W.shape[1] != d_in:
        raise ValueError("W's second dimension must be x's last")
    return rows, d_in, W.shape[0]


def _layer_out(x, W, out):
    rows, d_in, d_out = _layer_dims(x, W)
    z = torch.empty((*x.shape[:-1], d_out), dtype=torch.bfloat16, device=x.device) if out is None else out
    _check_out(z, "out", torch.bfloat16, rows * d_out, x.device)
    return rows, d_in, d_out, z


def grkan_layer_forward(x: torch.Tensor, A: torch.Tensor, B: torch.Tensor, W: torch.Tensor,
                        n_groups: int = 8, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """z = F(x) W^T, the GR-KAN layer with F fused into the matrix product
    (``grkan_layer_forward``); bf16 x [..., d_in], W [d_out, d_in]."""
    _check_coefs(A, B, n_groups, x.device)
    rows, d_in, d_out, z = _layer_out(x, W, out)
    st = load_library().grkan_layer_forward(_ptr(x), _ptr(A), _ptr(B), _ptr(W), _ptr(z), rows, d_in,
                                            d_out, n_groups, ctypes.c_void_p(_stream(stream)))
    if st != GRKAN_OK:
        raise GRKANError(st, "grkan_layer_forward")
    return z


def grkan_layer_forward_workspace_size(rows: int, d_in: int, d_out: int, n_groups: int = 8) -> int:
    return int(load_library().grkan_layer_forward_workspace_size(rows, d_in, d_out, n_groups))


def grkan_layer_forward_ws(x: torch.Tensor, A: torch.Tensor, B: torch.Tensor, W: torch.Tensor,
                           n_groups: int = 8, out: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """z = F(x) W^T by ``grkan_layer_forward_ws``: the fused or the unfused form, whichever the
    library takes for the shape (same bits); the workspace is allocated here when not given."""
    _check_coefs(A, B, n_groups, x.device)
    rows, d_in, d_out, z = _layer_out(x, W, out)
    lib = load_library()
    need = lib.grkan_layer_forward_workspace_size(rows, d_in, d_out, n_groups)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsp, wsn = _workspace(workspace, x.device)
    st = lib.grkan_layer_forward_ws(_ptr(x), _ptr(A), _ptr(B), _ptr(W), _ptr(z), rows, d_in, d_out, n_groups,
                                    wsp, wsn, ctypes.c_void_p(_stream(stream)))
    if st != GRKAN_OK:
        raise GRKANError(st, "grkan_layer_forward_ws")
    return z


def grkan_linear_forward(y: torch.Tensor, W: torch.Tensor, out: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    """z = y W^T on the same matrix-core kernel (``grkan_linear_forward``)."""
    rows, d_in, d_out, z = _layer_out(y, W, out)
    st = load_library().grkan_linear_forward(_ptr(y), _ptr(W), _ptr(z), rows, d_in, d_out,
                                             ctypes.c_void_p(_stream(stream)))
    if st != GRKAN_OK:
        raise GRKANError(st, "grkan_linear_forward")
    return z


def grkan_layer_backward_workspace_size(rows: int, d_in: int, d_out: int, n_groups: int = 8) -> int:
    return int(load_library().grkan_layer_backward_workspace_size(rows, d_in, d_out, n_groups))


def grkan_layer_backward(x: torch.Tensor, dz: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                         W: torch.Tensor, n_groups: int = 8, dx: torch.Tensor | None = None,
                         dA: torch.Tensor | None = None, dB: torch.Tensor | None = None,
                         dW: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         stream=None):
    """(dx, dA, dB, dW) of the GR-KAN layer (``grkan_layer_backward``): bf16 x [..., d_in],
    dz [..., d_out], W [d_out, d_in]; dx bf16, dA / dB / dW fp32."""
    _check_coefs(A, B, n_groups, x.device)
    rows, d_in, d_out = _layer_dims(x, W)
    _check_out(dz, "dz", torch.bfloat16, rows * d_out, x.device)
    dx, dA, dB = _grad_outputs(x, n_groups, GRKAN_M, GRKAN_N, dx, dA, dB)
    dW = torch.empty((d_out, d_in), dtype=torch.float32, device=x.device) if dW is None else dW
    _check_out(dW, "dW", torch.float32, d_out * d_in, x.device)
    lib = load_library()
    need = lib.grkan_layer_backward_workspace_size(rows, d_in, d_out, n_groups)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsp, wsn = _workspace(workspace, x.device)
    st = lib.grkan_layer_backward(_ptr(x), _ptr(dz), _ptr(A), _ptr(B), _ptr(W), _ptr(dx), _ptr(dA), _ptr(dB),
                                  _ptr(dW), rows, d_in, d_out, n_groups, wsp, wsn,
                                  ctypes.c_void_p(_stream(stream)))
    if st != GRKAN_OK:
        raise GRKANError(st, "grkan_layer_backward")
    return dx, dA, dB, dW


CHEBY_DEGREE = 7


def _cheby_dims(x, C, degree):
    if x.dtype != torch.bfloat16 or C.dtype != torch.bfloat16:
        raise TypeError("the Chebyshev-KAN layer takes bfloat16 x and C")
    _on_gpu(x)
    rows, d_in = _rows_d(x)
    if C.dim() != 3 or C.shape[1] != d_in or C.shape[2] != degree + 1 or not C.is_contiguous() \
            or C.device != x.device:
        raise ValueError("C must be a contiguous [d_out, d_in, degree + 1] tensor on x's device")
    return rows, d_in, C.shape[0]


def grkan_chebykan_forward(x: torch.Tensor, C: torch.Tensor, degree: int = CHEBY_DEGREE,
                           out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = sum_i sum_k C[o, i, k] T_k(tanh x_i) (``grkan_chebykan_forward``), bf16."""
    rows, d_in, d_out = _cheby_dims(x, C, degree)
    y = torch.empty((*x.shape[:-1], d_out), dtype=torch.bfloat16, device=x.device) if out is None else out
    _check_out(y, "out", torch.bfloat16, rows * d_out, x.device)
    st = load_library().grkan_chebykan_forward(_ptr(x), _ptr(C), _ptr(y), rows, d_in, d_out, degree,
                                               ctypes.c_void_p(_stream(stream)))
    if st != GRKAN_OK:
        raise GRKANError(st, "grkan_chebykan_forward")
    return y


def grkan_chebykan_backward_workspace_size(rows: int, d_in: int, d_out: int, degree: int = CHEBY_DEGREE) -> int:
    return int(load_library().grkan_chebykan_backward_workspace_size(rows, d_in, d_out, degree))


def grkan_chebykan_backward(x: torch.Tensor, dy: torch.Tensor, C: torch.Tensor, degree: int = CHEBY_DEGREE,
                            dx: torch.Tensor | None = None, dC: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None, stream=None):
    """(dx, dC) of the Chebyshev-KAN layer (``grkan_chebykan_backward``): dx bf16, dC fp32."""
    rows, d_in, d_out = _cheby_dims(x, C, degree)
    _check_out(dy, "dy", torch.bfloat16, rows * d_out, x.device)
    if dx is None:
        dx = torch.empty_like(x)
    _check_out(dx, "dx", torch.bfloat16, x.numel(), x.device)
    dC = torch.empty(C.shape, dtype=torch.float32, device=x.device) if dC is None else dC
    _check_out(dC, "dC", torch.float32, C.numel(), x.device)
    lib = load_library()
    need = lib.grkan_chebykan_backward_workspace_size(rows, d_in, d_out, degree)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsp, wsn = _workspace(workspace, x.device)
    st = lib.grkan_chebykan_backward(_ptr(x), _ptr(dy), _ptr(C), _ptr(dx), _ptr(dC), rows, d_in, d_out, degree,
                                     wsp, wsn, ctypes.c_void_p(_stream(stream)))
    if st != GRKAN_OK:
        raise GRKANError(st, "grkan_chebykan_backward")
    return dx, dC


def grkan_query_launch(rows: int, d: int, n_groups: int, io: int, pass_: int) -> dict:
    """Launch geometry on the current device (pass_ 0 = forward, 1 = backward,
    2 = backward with GRKAN_BLOCK_ATOMIC)."""
    out = grkan_launch_t()
    st = load_library().grkan_query_launch(rows, d, n_groups, io, pass_, ctypes.byref(out))
    if st != GRKAN_OK:
        raise GRKANError(st, "grkan_query_launch")
    return {f: getattr(out, f) for f, _ in grkan_launch_t._fields_}


def grkan_pau_query_launch(rows: int, d: int, n_groups: int, m: int, n: int, io: int,
                           pass_: int) -> dict:
    """grkan_query_launch for degrees (m, n)."""
    out = grkan_launch_t()
    st = load_library().grkan_pau_query_launch(rows, d, n_groups, m, n, io, pass_, ctypes.byref(out))
    if st != GRKAN_OK:
        raise GRKANError(st, "grkan_pau_query_launch")
    return {f: getattr(out, f) for f, _ in grkan_launch_t._fields_}


class GRKANFunction(torch.autograd.Function):
    """Autograd wrapper: forward by grkan_forward, backward by grkan_backward."""

    @staticmethod
    def forward(ctx, x, A, B, n_groups=8):
        ctx.save_for_backward(x, A, B)
        ctx.n_groups = n_groups
        return grkan_forward(x.contiguous(), A.contiguous(), B.contiguous(), n_groups)

    @staticmethod
    def backward(ctx, dy):
        x, A, B = ctx.saved_tensors
        dx, dA, dB = grkan_backward(x.contiguous(), dy.contiguous(), A.contiguous(), B.contiguous(),
                                    ctx.n_groups)
        return dx, dA.view_as(A), dB.view_as(B), None
