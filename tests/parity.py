"""Comparison rules between the HIP path and the fp64 oracle.

Tolerances (fixed here, used by every parity test):

* Y and dX, elementwise, fp32 I/O:  |gpu - ref| <= 1e-5 * max(|ref|, M)
  where M is the oracle's first-order rounding scale of that element (sums of
  the absolute values of every term, see oracle/grkan_oracle.c).  For
  elements away from zeros of the result, M ~ |ref| and this is the plain
  relative 1e-5; next to a zero of P (or of dX) a relative test cannot hold
  for any fp32 evaluation, and the scale M takes over.
* bf16 I/O: the same plus half a bf16 ulp of the returned value (the
  kernel rounds an fp32 result to nearest-even bf16).
* dA and dB: |gpu - ref| <= 1e-4 * max(|ref|, 1e-2 * ||t||_2) + 1e-6, with
  ||t||_2 the L2 norm of the group's terms.  Rounding every term in fp32
  leaves an error of order 2^-24 * ||t||_2 whatever the summation; a sum
  that cancels to |ref| << ||t||_2 is therefore compared at 1e-6 ||t||_2,
  about 17 units of that floor.
* dA and dB in the deterministic scheme at GR-KAN's degrees (5, 4), the five
  GR-KAN workloads included: additionally the literal rule of the task,
  |gpu - ref| <= max(1e-4 |ref|, 1e-6), asserted (``literal=True``).
* dA and dB at the PAU degree pairs (6, 5) and (7, 6) only: plus
  8 * 2^-24 * ||m||_2 with ||m||_2 the L2 norm of the terms' first-order
  rounding scales (oracle: magsq).  Each term is evaluated from an fp32 Q
  whose rounding error is relative to Qabs, the sum of |b_j x^j|, not to |Q|;
  next to a root of Q with large terms (degree-5 and -6 denominators at
  |x| ~ 3) one element's term can be off by far more than 2^-24 |t|, and no
  fp32 evaluation avoids that.  At GR-KAN's degrees this allowance is not
  needed and not given: on the committed full-size sums of the five GR-KAN
  workloads it would exceed the 1e-6 ||t||_2 floor (by up to ~100x on dB),
  i.e. it would widen the bound where nothing requires it.
* dA and dB of the comparison scheme GRKAN_BLOCK_ATOMIC (one fp32 atomic add
  per coefficient per workgroup, the pages' Algorithm 2): the above plus
  8 * 2^-24 * sqrt(n) * ||t||_2 for n workgroup partials added in fp32 in an
  arbitrary order.  Recursive fp32 summation of n zero-mean partials whose
  running sum wanders on the scale of ||t||_2 leaves an error of about
  2^-24 * sqrt(n / 2) * ||t||_2; this scheme does not meet the default
  scheme's bound at large n, which is the pages' point about atomics.
* The layer backward (oracle/layer.py): dx, dA, dB by the activation's
  rules above plus the allowances for elements whose upstream bf16 rounding
  of dz W is not unique (dx_amb, dA_amb, dB_amb); dW by the dA / dB rule
  (its terms dz bf16(F) are exact in fp32) plus dW_amb.
* The bf16 GR-KAN layer z = bf16(F(x)) W^T (oracle/layer.py):
  |gpu - ref| <= amb + gamma * mag + ulp_bf16(|ref| + amb + gamma * mag),
  gamma = K * 2^-24.  amb covers elements whose bf16 rounding of F is not
  unique at fp32 accuracy (either neighbour is a correct operand), gamma *
  mag bounds fp32 accumulation of K exact bf16 products (mag = sum of their
  absolute values), and one bf16 unit covers the rounding of z.
"""
from __future__ import annotations

import numpy as np

REL_ELEM = 1e-5
REL_SUM = 1e-4
SUM_FLOOR = 1e-2
ABS_SUM = 1e-6


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(v, dtype=np.float64))
    out = np.zeros_like(a)
    nz = a > 0
    out[nz] = 2.0 ** (np.floor(np.log2(a[nz])) - 7)
    return out


def elem_tol(ref: np.ndarray, mag: np.ndarray, gpu: np.ndarray, io: str = "f32") -> np.ndarray:
    tol = REL_ELEM * np.maximum(np.abs(ref), mag)
    if io == "bf16":
        tol = tol + 0.5 * ulp_bf16(gpu)
    return tol


def check_elem(name: str, gpu: np.ndarray, ref: np.ndarray, mag: np.ndarray, io: str = "f32") -> dict:
    gpu = np.asarray(gpu, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    mag = np.asarray(mag, dtype=np.float64).ravel()
    err = np.abs(gpu - ref)
    tol = elem_tol(ref, mag, gpu, io)
    bad = ~(err <= tol)
    literal = int(np.sum(err > REL_ELEM * np.abs(ref) + (0.5 * ulp_bf16(gpu) if io == "bf16" else 0)))
    stats = {"n": int(gpu.size), "bad": int(bad.sum()), "literal_rel_fail": literal,
             "max_err_over_tol": float(np.max(err / np.maximum(tol, 1e-300))) if gpu.size else 0.0}
    if bad.any():
        i = np.flatnonzero(bad)[:8]
        raise AssertionError(f"{name}: {stats['bad']}/{gpu.size} outside tolerance; first at {i.tolist()}: "
                             f"gpu={gpu[i].tolist()} ref={ref[i].tolist()} tol={tol[i].tolist()}")
    return stats


TERM_ROUNDING = 8 * 2.0 ** -24
# Degree pairs whose dA / dB comparison carries the TERM_ROUNDING allowance (see above): the
# ones where fp32 terms next to a root of a high-degree Q were measured to need it.
TERM_ROUNDING_PAIRS = {(6, 5), (7, 6)}


def term_mag(m: int, n: int, mag):
    """The rounding-scale norms to pass as ``mag`` for degrees (m, n): only for the pairs that
    need the allowance, else None."""
    return mag if (m, n) in TERM_ROUNDING_PAIRS else None


def literal_tol(ref: np.ndarray) -> np.ndarray:
    """The task's literal dA / dB rule: rel 1e-4 with an absolute floor of 1e-6."""
    return np.maximum(REL_SUM * np.abs(ref), ABS_SUM)


def sum_tol(ref: np.ndarray, norm: np.ndarray, mag=None) -> np.ndarray:
    tol = REL_SUM * np.maximum(np.abs(ref), SUM_FLOOR * norm) + ABS_SUM
    if mag is not None:
        tol = tol + TERM_ROUNDING * np.asarray(mag, dtype=np.float64)
    return tol


def check_sums(name: str, gpu: np.ndarray, ref: np.ndarray, norm: np.ndarray,
               atomic_adds: int = 0, mag=None, extra=None, literal: bool = False) -> dict:
    """``mag``: L2 norm of the terms' rounding scales (oracle ``mA`` / ``mB``), given only for the
    degree pairs in TERM_ROUNDING_PAIRS.  ``literal``: also assert the literal rule."""
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ref)
    tol = sum_tol(ref, norm, mag)
    if extra is not None:
        tol = tol + extra
    if atomic_adds:
        tol = tol + 8 * 2.0 ** -24 * np.sqrt(atomic_adds) * norm
    bad = ~(err <= tol)
    lit_bad = ~(err <= literal_tol(ref))
    stats = {"bad": int(bad.sum()), "literal_fail": int(lit_bad.sum()),
             "max_err_over_literal": float(np.max(err / literal_tol(ref))) if err.size else 0.0,
             "max_rel": float(np.max(err / np.maximum(np.abs(ref), 1e-300))),
             "max_err_over_norm": float(np.max(err / np.maximum(norm, 1e-300)))}
    if bad.any():
        idx = np.argwhere(bad)[:8].tolist()
        raise AssertionError(f"{name}: {stats['bad']} coefficients outside tolerance at {idx}: "
                             f"gpu={gpu[bad][:8].tolist()} ref={ref[bad][:8].tolist()} "
                             f"tol={tol[bad][:8].tolist()}")
    if literal and lit_bad.any():
        idx = np.argwhere(lit_bad)[:8].tolist()
        raise AssertionError(f"{name}: {int(lit_bad.sum())} coefficients fail the literal rule "
                             f"(rel 1e-4, abs 1e-6) at {idx}: gpu={gpu[lit_bad][:8].tolist()} "
                             f"ref={ref[lit_bad][:8].tolist()}")
    return stats


def check_layer(name: str, gpu: np.ndarray, ref: dict, k: int) -> dict:
    """Elementwise layer check; returns statistics, raises on a failure."""
    gpu = np.asarray(gpu, dtype=np.float64)
    z, amb, mag = ref["z"], ref["amb"], ref["mag"]
    slack = amb + k * 2.0 ** -24 * mag
    tol = slack + ulp_bf16(np.abs(z) + slack)
    err = np.abs(gpu - z)
    bad = err > tol
    st = {"n": int(gpu.size), "fail": int(np.count_nonzero(bad)),
          "max_err_over_tol": float(np.max(err / np.maximum(tol, 1e-300))) if gpu.size else 0.0}
    if st["fail"]:
        i = int(np.flatnonzero(bad.ravel())[0])
        raise AssertionError(f"{name}: {st['fail']} of {st['n']} outside tolerance; first at {i}: "
                             f"gpu {gpu.ravel()[i]!r} ref {z.ravel()[i]!r} tol {tol.ravel()[i]!r}")
    return st


def check_elem_extra(name: str, gpu: np.ndarray, ref: np.ndarray, mag: np.ndarray, extra: np.ndarray,
                     io: str = "f32") -> dict:
    """check_elem with an extra allowance per element."""
    gpu = np.asarray(gpu, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    tol = elem_tol(ref, np.asarray(mag, dtype=np.float64).ravel(), gpu, io) + np.asarray(extra).ravel()
    err = np.abs(gpu - ref)
    bad = ~(err <= tol)
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{name}: {int(bad.sum())} of {gpu.size} outside tolerance; first at {i}: "
                             f"gpu {gpu[i]!r} ref {ref[i]!r} tol {tol[i]!r}")
    return {"n": int(gpu.size)}
