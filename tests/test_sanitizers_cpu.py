"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer builds, run on the CPU.

* The C oracle (oracle/grkan_oracle.c, built with gcc) driven by
  tests/sanitize/oracle_main.c: every entry point over every degree pair up to
  the limit, edge shapes, rejected arguments and special values.
* The library's host code (every translation unit, built with hipcc and the
  sanitizers on the host side only) driven by tests/sanitize/abi_main.c: every
  C-ABI entry point with arguments it must reject, and the host-only queries
  over many shapes.  Validation precedes every HIP call, so no GPU is needed.

Either run aborts with a non-zero status on the first sanitizer report.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "gr_kan_rational_amd", "csrc")
# the sanitizers stay on the host side of every hipcc line
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
SAN_GCC = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _env(leaks: bool) -> dict:
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = f"detect_leaks={1 if leaks else 0}:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    return env


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise AssertionError(f"{' '.join(map(str, cmd))} failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}")
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=gnu11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", *SAN_GCC,
          os.path.join(ROOT, "oracle", "grkan_oracle.c"), os.path.join(HERE, "oracle_main.c"), "-lm", "-o", exe])
    r = _run([exe], env=_env(leaks=True), timeout=300)
    assert "oracle sanitizer run: ok" in r.stdout


def test_abi_host_code_under_sanitizers(tmp_path):
    from gr_kan_rational_amd import _build

    try:
        cc = _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    common = [f"--offload-arch={_build.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    jobs = []
    for name, extra, obj in _build.units():
        jobs.append([cc, *common, *SAN_HOST, *extra, "-c", os.path.join(CSRC, name), "-o", str(tmp_path / obj)])
    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda c: _run(c, timeout=600), jobs))
    main_o = str(tmp_path / "abi_main.o")
    _run(["gcc", "-std=gnu11", "-O1", "-g", *SAN_GCC, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
          "-I", "/opt/rocm/include", "-c", os.path.join(HERE, "abi_main.c"), "-o", main_o])
    exe = str(tmp_path / "abi_san")
    objs = [str(tmp_path / obj) for _, _, obj in _build.units()]
    _run([cc, f"--offload-arch={_build.ARCH}", *SAN_HOST, main_o, *objs, "-o", exe], timeout=600)
    # the HIP runtime's own allocations are not this library's: leaks are not reported here
    r = _run([exe], env=_env(leaks=False), timeout=300)
    assert "ABI sanitizer run: ok" in r.stdout
