"""Every element of a full-size forward / backward against the fp64 oracle.

The GPU outputs are copied to the host once, in their own dtype (fp32 or the
bf16 bit patterns); the rows are then cut into chunks that worker threads
evaluate with the oracle (one thread each, so the oracle's own chunking is
unchanged) and compare with ``parity.check_elem``.  Only chunk-sized fp64
buffers exist at any time.  Statistics are summed over the chunks; the first
failing chunk raises.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import oracle as orc
import parity

CHUNK_ELEMS = 1 << 20


def host_raw(t: torch.Tensor) -> np.ndarray:
    """Host copy of a device tensor in its own bits: float32, or bf16 as uint16."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def decode(a: np.ndarray, io: str) -> np.ndarray:
    if io == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a


def compare_all(name: str, w, inp: dict, y: torch.Tensor, dx: torch.Tensor, log=print) -> dict:
    """Y and dX of workload ``w`` (inputs ``inp`` from synth.make_inputs), every element."""
    d = w.d
    rows = w.rows
    yh = host_raw(y).reshape(rows, d)
    dxh = host_raw(dx).reshape(rows, d)
    x2 = inp["x"].reshape(rows, d)
    dy2 = inp["dy"].reshape(rows, d)
    step = max(1, CHUNK_ELEMS // d)
    starts = list(range(0, rows, step))

    def work(r0):
        r1 = min(rows, r0 + step)
        ref = orc.run(x2[r0:r1], inp["A"], inp["B"], w.n_groups, dy=dy2[r0:r1], io=w.io,
                      nthreads=1, m=w.m, n=w.n)
        sy = parity.check_elem(f"{name} Y rows {r0}..{r1}", decode(yh[r0:r1], w.io), ref["y"], ref["ymag"], w.io)
        sd = parity.check_elem(f"{name} dX rows {r0}..{r1}", decode(dxh[r0:r1], w.io), ref["dx"], ref["dxmag"],
                               w.io)
        return sy, sd

    tot = {"Y": {"n": 0, "literal_rel_fail": 0, "max_err_over_tol": 0.0},
           "dX": {"n": 0, "literal_rel_fail": 0, "max_err_over_tol": 0.0}}
    with ThreadPoolExecutor(orc.threads()) as ex:
        for sy, sd in ex.map(work, starts):
            for key, s in (("Y", sy), ("dX", sd)):
                t = tot[key]
                t["n"] += s["n"]
                t["literal_rel_fail"] += s["literal_rel_fail"]
                t["max_err_over_tol"] = max(t["max_err_over_tol"], s["max_err_over_tol"])
    assert tot["Y"]["n"] == w.elements and tot["dX"]["n"] == w.elements
    log(f"{name}: every element compared: {tot}")
    return tot
