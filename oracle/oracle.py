"""fp64 CPU oracle for the GR-KAN safe Pade activation (forward and backward).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this module.  The HIP
library never loads it, and it shares no code with the HIP path.

The arithmetic lives in ``grkan_oracle.c`` (plain C, fp64; see its header for
the definition being computed and the passages of the pages it follows).
This wrapper only:

* converts fp32 / bf16 inputs to their exact fp64 values,
* cuts the rows into fixed chunks and runs the C routine on them from a
  thread pool (each chunk sums its rows in index order; the chunk sums are
  combined exactly with ``math.fsum``),
* gathers sampled elements for the one-by-one checks at full size.

Every function here is pinned by the ``not gpu`` tests in
``tests/test_oracle_pins.py`` (closed forms, library routines, symbolic
differentiation, finite differences, brute-force sums).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "grkan_oracle.c")
# GRKAN_ORACLE_LIB names another build of grkan_oracle.c to load instead (the
# mutation tests point it at copies with a planted mistake); never built here.
_BUILT = os.path.join(_HERE, "libgrkan_oracle.so")
_LIB_ENV = os.environ.get("GRKAN_ORACLE_LIB")
_LIB = _LIB_ENV or _BUILT

M, N = 5, 4             # GR-KAN's degrees: numerator a_0..a_5, denominator b_1..b_4
NA, NB = M + 1, N
NK = NA + NB
# record layout of grkan_oracle_point (kept in step with the C enum): six
# scalars, then the m+1 numerator terms and the n denominator terms, then the
# first-order rounding scale of each of those terms in the same order
F, DX, FMAG, DXMAG, SIGN, DEN, T = 0, 1, 2, 3, 4, 5, 6


def layout(m: int = M, n: int = N):
    """(first numerator term, first denominator term, record length) for degrees (m, n);
    the rounding scale of the term at column c sits at column c + m + 1 + n."""
    return T, T + m + 1, T + 2 * (m + 1 + n)


TA, TB, NOUT = layout()
MAXDEG = 15

_CHUNK_ELEMS = 1 << 16


def build(force: bool = True) -> str:
    """Compile ``grkan_oracle.c`` with gcc into ``libgrkan_oracle.so``."""
    if not force and os.path.exists(_BUILT):
        return _BUILT
    tmp = _BUILT + ".tmp"
    cmd = ["gcc", "-std=gnu11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _BUILT)
    return _BUILT


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB):
            if _LIB_ENV:
                raise FileNotFoundError(f"GRKAN_ORACLE_LIB={_LIB_ENV} does not exist")
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_long)
        ci = ctypes.c_int
        lib.grkan_oracle_point.argtypes = [ctypes.c_double, ctypes.c_double, ci, ci, dp, dp, dp]
        lib.grkan_oracle_point.restype = None
        lib.grkan_oracle_rows.argtypes = [dp, dp, ctypes.c_long, ctypes.c_long, ci, ci, ci,
                                          dp, dp, dp, dp, dp, dp, dp, dp, dp]
        lib.grkan_oracle_rows.restype = ci
        lib.grkan_oracle_points.argtypes = [dp, dp, lp, ctypes.c_long, ctypes.c_long,
                                            ci, ci, ci, dp, dp, dp]
        lib.grkan_oracle_points.restype = ci
        lib.grkan_oracle_nout.argtypes = [ci, ci]
        lib.grkan_oracle_nout.restype = ci
        if any(lib.grkan_oracle_nout(m, n) != layout(m, n)[2] for m, n in ((5, 4), (0, 0), (7, 3))):
            raise RuntimeError("oracle library record layout does not match oracle.py")
        _lib_handle = lib
    return _lib_handle


def threads() -> int:
    """Host threads the oracle uses: the CPU share the machine declares for this process through
    OMP_NUM_THREADS when it sets one (a shared GPU host allots each GPU's jobs a share of its
    cores), else every CPU this process may run on."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def to_f64(a: np.ndarray, io: str = "f32") -> np.ndarray:
    """Exact fp64 value of an fp32 array, or of a bf16 array stored as uint16 bits."""
    if io == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 data must be given as its uint16 bit patterns")
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if io == "f32":
        if a.dtype != np.float32:
            raise TypeError("f32 data must be float32")
        return a.astype(np.float64)
    raise ValueError(f"unknown io dtype {io!r}")


def _load_f64(dst: np.ndarray, src: np.ndarray, io: str, local) -> np.ndarray:
    """to_f64 into a preallocated buffer (no temporaries)."""
    if io == "bf16":
        if src.dtype != np.uint16:
            raise TypeError("bf16 data must be given as its uint16 bit patterns")
        u = getattr(local, "u32", None)
        if u is None or u.size < src.size:
            u = np.empty(src.size, dtype=np.uint32)
            local.u32 = u
        u = u[:src.size]
        np.copyto(u, src)
        np.left_shift(u, 16, out=u)
        np.copyto(dst, u.view(np.float32))
    elif io == "f32":
        if src.dtype != np.float32:
            raise TypeError("f32 data must be float32")
        np.copyto(dst, src)
    else:
        raise ValueError(f"unknown io dtype {io!r}")
    return dst


def _degrees(m, n):
    if not (0 <= m <= MAXDEG and 0 <= n <= MAXDEG):
        raise ValueError(f"degrees (m, n) = ({m}, {n}) outside 0..{MAXDEG}")


def _coef(A, B, n_groups, m=M, n=N):
    _degrees(m, n)
    A = np.ascontiguousarray(np.asarray(A, dtype=np.float64).reshape(n_groups, m + 1))
    B = np.ascontiguousarray(np.asarray(B, dtype=np.float64).reshape(n_groups, n))
    if n == 0:  # keep a valid pointer for an empty denominator
        B = np.zeros((n_groups, 1), dtype=np.float64)
    return A, B


def point(x: float, dy: float, a, b, m: int = M, n: int = N) -> np.ndarray:
    """One element: the record of grkan_oracle_point (a: m+1 values, b: n values)."""
    A, B = _coef(a, b, 1, m, n)
    out = np.zeros(layout(m, n)[2], dtype=np.float64)
    _lib().grkan_oracle_point(float(x), float(dy), m, n, _ptr(A), _ptr(B), _ptr(out))
    return out


def run(x, A, B, n_groups: int, dy=None, io: str = "f32", elements: bool = True,
        nthreads: int | None = None, m: int = M, n: int = N) -> dict:
    """Forward (and backward when ``dy`` is given) over a whole [..., d] tensor.

    Degrees (m, n): A is [n_g, m+1], B is [n_g, n].  Returns a dict with fp64
    arrays shaped like ``x`` for ``y``, ``ymag`` and, with ``dy``, ``dx``,
    ``dxmag`` (only when ``elements``), and always, with ``dy``, ``dA``
    [n_g, m+1], ``dB`` [n_g, n], the L2 norms of their terms ``nA``, ``nB``
    and the L2 norms of their terms' rounding scales ``mA``, ``mB`` (same
    shapes).
    """
    nk = m + 1 + n
    shape = x.shape
    d = shape[-1]
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    x2 = x.reshape(rows, d)
    dy2 = None if dy is None else dy.reshape(rows, d)
    A64, B64 = _coef(A, B, n_groups, m, n)
    lib = _lib()
    res = {}
    if elements:
        res["y"] = np.empty((rows, d), dtype=np.float64)
        res["ymag"] = np.empty((rows, d), dtype=np.float64)
        if dy is not None:
            res["dx"] = np.empty((rows, d), dtype=np.float64)
            res["dxmag"] = np.empty((rows, d), dtype=np.float64)
    step = max(1, _CHUNK_ELEMS // d)
    starts = list(range(0, rows, step))
    nchunk = len(starts)
    sums = np.zeros((nchunk, n_groups * nk), dtype=np.float64)
    sumsq = np.zeros((nchunk, n_groups * nk), dtype=np.float64)
    magsq = np.zeros((nchunk, n_groups * nk), dtype=np.float64)

    local = threading.local()

    def scratch(name, n):
        buf = getattr(local, name, None)
        if buf is None or buf.size < n:
            buf = np.empty(n, dtype=np.float64)
            setattr(local, name, buf)
        return buf[:n]

    def work(ci):
        r0 = starts[ci]
        r1 = min(rows, r0 + step)
        ne = (r1 - r0) * d
        xc = _load_f64(scratch("x", ne), x2[r0:r1].reshape(-1), io, local)
        dyc = None
        if dy2 is not None:
            dyc = _load_f64(scratch("dy", ne), dy2[r0:r1].reshape(-1), io, local)
        outs = {k: res[k][r0:r1] for k in res}  # row slices of C-contiguous arrays
        sp = _ptr(sums[ci]) if dy is not None else None
        sq = _ptr(sumsq[ci]) if dy is not None else None
        mq = _ptr(magsq[ci]) if dy is not None else None
        rc = lib.grkan_oracle_rows(_ptr(xc), _ptr(dyc), r1 - r0, d, n_groups, m, n,
                                   _ptr(A64), _ptr(B64), _ptr(outs.get("y")),
                                   _ptr(outs.get("ymag")), _ptr(outs.get("dx")),
                                   _ptr(outs.get("dxmag")), sp, sq, mq)
        if rc != 0:
            raise ValueError("oracle rejected the shape")

    nt = nthreads or threads()
    if nt == 1 or nchunk == 1:
        for ci in range(nchunk):
            work(ci)
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(work, range(nchunk)))

    for k in list(res):
        res[k] = res[k].reshape(shape)
    if dy is not None:
        tot = np.array([math.fsum(sums[:, k]) for k in range(n_groups * nk)]).reshape(n_groups, nk)
        tot2 = np.array([math.fsum(sumsq[:, k]) for k in range(n_groups * nk)]).reshape(n_groups, nk)
        tot3 = np.array([math.fsum(magsq[:, k]) for k in range(n_groups * nk)]).reshape(n_groups, nk)
        nrm = np.sqrt(tot2)
        mag = np.sqrt(tot3)
        res["dA"], res["dB"] = tot[:, :m + 1].copy(), tot[:, m + 1:].copy()
        res["nA"], res["nB"] = nrm[:, :m + 1].copy(), nrm[:, m + 1:].copy()
        res["mA"], res["mB"] = mag[:, :m + 1].copy(), mag[:, m + 1:].copy()
    return res


def points(x, A, B, n_groups: int, flat_idx, dy=None, io: str = "f32", m: int = M,
           n: int = N) -> np.ndarray:
    """Records [n_el, layout(m, n)[2]] for the elements at flat indices ``flat_idx`` of ``x``."""
    d = x.shape[-1]
    flat_idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    xv = np.ascontiguousarray(to_f64(x.reshape(-1)[flat_idx], io))
    dyv = None if dy is None else np.ascontiguousarray(to_f64(dy.reshape(-1)[flat_idx], io))
    A64, B64 = _coef(A, B, n_groups, m, n)
    out = np.empty((flat_idx.size, layout(m, n)[2]), dtype=np.float64)
    rc = _lib().grkan_oracle_points(_ptr(xv), _ptr(dyv),
                                    flat_idx.ctypes.data_as(ctypes.POINTER(ctypes.c_long)),
                                    flat_idx.size, d, n_groups, m, n, _ptr(A64), _ptr(B64),
                                    _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the shape")
    return out
