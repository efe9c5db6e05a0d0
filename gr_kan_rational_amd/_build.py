"""Build libgrkan.so (gfx950) in-tree with hipcc.

Every translation unit is compiled for gfx950 only, with packed-FP32
instruction selection disabled, then linked into ``libgrkan.so`` next to this
file.  The kernel source is compiled once per (numerator, denominator) degree
pair listed in ``GRKAN_FOR_EACH_DEGREE`` (csrc/grkan_launch.h).  The baseline kernel's translation unit is compiled with the compiler's
atomic optimizer off so that each lane's atomic stays a hardware atomic.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgrkan.so")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
]
LAUNCH_H = os.path.join(CSRC, "grkan_launch.h")


def degree_pairs() -> list[tuple[int, int]]:
    """The (m, n) pairs listed in GRKAN_FOR_EACH_DEGREE in grkan_launch.h."""
    text = open(LAUNCH_H).read()
    m = re.search(r"#define GRKAN_FOR_EACH_DEGREE\(X\)((?:\s*X\(\d+, \d+\))+)", text)
    if not m:
        raise RuntimeError("GRKAN_FOR_EACH_DEGREE not found in grkan_launch.h")
    return [(int(a), int(b)) for a, b in re.findall(r"X\((\d+), (\d+)\)", m.group(1))]


def units() -> list[tuple[str, list[str], str]]:
    """(source, extra flags, object name) of every translation unit."""
    out = [("grkan_api.hip", [], "grkan_api.o"),
           ("grkan_merge.hip", [], "grkan_merge.o"),
           ("grkan_layer.hip", [], "grkan_layer.o"),
           ("grkan_probe.hip", [], "grkan_probe.o"),
           ("grkan_naive.hip", ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"], "grkan_naive.o")]
    for m, n in degree_pairs():
        out.append(("grkan_kernels.hip", [f"-DGRKAN_M={m}", f"-DGRKAN_N={n}"], f"grkan_kernels_{m}_{n}.o"))
    return out


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    cc = hipcc()

    def compile_unit(item):
        name, extra, obj = item
        out = os.path.join(OBJ, obj)
        cmd = [cc, *COMMON, *extra, "-c", os.path.join(CSRC, name), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {name} {' '.join(extra)}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr)
        return out

    todo = units()
    with ThreadPoolExecutor(min(len(todo), max(1, os.cpu_count() or 1), 16)) as ex:
        objs = list(ex.map(compile_unit, todo))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
