"""Write the fp64 oracle's group sums for each full-size workload.

Output: tests/golden/<workload>.sums.json with dA, dB (the oracle's group sums
over the whole workload), nA, nB (L2 norms of the summed terms) and mA, mB
(L2 norms of the terms' rounding scales), as exact float reprs.  Calls only the oracle and the seeded input generator; the GPU
parity tests check that a fresh oracle run reproduces these files, and the
benchmark reads them to report the rounding error of the GPU reductions.

    python tests/golden/make_golden.py [workload ...]
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from gr_kan_rational_amd import synth  # noqa: E402
from oracle import oracle  # noqa: E402


def path_for(name: str) -> str:
    return os.path.join(HERE, f"{name}.sums.json")


def make(name: str) -> dict:
    w = synth.WORKLOADS[name]
    t0 = time.time()
    inp = synth.make_inputs(w)
    r = oracle.run(inp["x"], inp["A"], inp["B"], w.n_groups, dy=inp["dy"], io=w.io, elements=False,
                   m=w.m, n=w.n)
    out = {
        "workload": name,
        "shape": [w.batch, w.seq, w.d],
        "n_groups": w.n_groups,
        "degrees": [w.m, w.n],
        "io": w.io,
        "seed": w.seed,
        "source": "oracle/grkan_oracle.c via oracle.oracle.run (fp64 terms, long double row sums, "
                  "fsum over row chunks)",
        "dA": [[float(v) for v in row] for row in r["dA"]],
        "dB": [[float(v) for v in row] for row in r["dB"]],
        "nA": [[float(v) for v in row] for row in r["nA"]],
        "nB": [[float(v) for v in row] for row in r["nB"]],
        "mA": [[float(v) for v in row] for row in r["mA"]],
        "mB": [[float(v) for v in row] for row in r["mB"]],
    }
    with open(path_for(name), "w") as f:
        json.dump(out, f, indent=1)
    print(f"{name}: {time.time() - t0:.1f} s", flush=True)
    return out


if __name__ == "__main__":
    names = sys.argv[1:] or list(synth.WORKLOADS)
    for n in names:
        make(n)
