"""Benchmark: GR-KAN activation forward + backward throughput on one MI355X.

A step is one forward (grkan_forward) and one backward (grkan_backward,
deterministic two-stage reduction) of the group-rational activation over a
whole batch of synthetic activations, all resident in HBM before timing.
Default workload: KAT-B shape, fp32 [1024, 197, 768], 8 groups.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload kat-b]
                    [--mode deterministic|atomic] [--no-cpu-baseline] [--no-naive]
                    [--inflate 2,4,8|none]

Prints one JSON line.  `value` is elements per second of the whole step
(E / step time, K back-to-back steps between two HIP events); `roofline`
rates the dominant kernel -- the backward call (main kernel + merge) -- by
its algorithmic bytes (read x and dy, write dx: 12 B per fp32 element) over
its average duration in a loop of K back-to-back backward calls, timed with
HIP events on the stream it runs on.  Workloads whose tensors would fit the
256 MB Infinity Cache (KAT-T: 58 MB per backward) rotate copies of their
inputs in distinct buffers, call by call, so that every call streams from
HBM; a second timing with the cache flushed before each call (a 512 MB write
outside the events) cross-checks it.  `detail.stream_probe_GBps` is the
measured ceiling of the backward's traffic: grkan_stream_probe (two reads,
one write, no arithmetic) over the same buffers.  A bf16-I/O backward does the
same arithmetic per element on half the bytes and is bound by its vector-ALU
work: its `roofline` rates it against the vector-ALU peak instead (lane
operations the method needs per element over the call's duration), with the
HBM figures under `roofline.hbm`.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same
workload.  `detail` adds the forward's figures, the atomic-mode and naive
per-element-atomic backward times, the rounding error of each backward
reduction against the oracle's fp64 group sums (tests/golden), and the
FLOP-inflation probe: forward and backward times with each element's
arithmetic repeated 2, 4 and 8 times (same outputs, same memory traffic).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
# Vector-ALU peak in lane operations per second (an FMA counts once): the published fp32
# vector rate, 157.3 TFLOP/s = 256 CUs x 128 FMA lanes per clock x 2 x 2.4 GHz, halved.
VALU_PEAK_TOPS = 256 * 128 * 2.4e9 / 1e12
MALL_BYTES = 256 << 20  # MI355X Infinity Cache
MALL_DEFEAT_BYTES = 8 * MALL_BYTES  # rotated input sets hold at least this much
MAX_SETS = 64
FLUSH_BYTES = 2 * MALL_BYTES  # read before each call of the flushed cross-check
PROFILES = os.path.join(ROOT, "profiles")
GOLDEN = os.path.join(ROOT, "tests", "golden")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("grkan_kernels.hip", "grkan_device.h", "grkan_qsign.h", "grkan_api.hip", "grkan_merge.hip"):
        with open(os.path.join(ROOT, "gr_kan_rational_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def backward_valu_ops_per_element(m: int, n: int, io: str) -> int:
    """Vector-ALU operations one backward element needs in these kernels (degrees m, n >= 1):
    bf16 unpack of x and dy, powers x^2..x^max(m,n), P, P', Q in fp64 (n - 1 FMAs, x q, two
    conversions), Q', D and 1/D, w, F, v, s v, w P', dX, the sign guard (one FMA, one compare)
    and the m + 1 + n gradient terms -- 44 for GR-KAN's (5, 4) with bf16 I/O."""
    return ((2 if io == "bf16" else 0) + (max(m, n) - 1) + m + (m - 1) + (n + 2) + (n - 1) + 2 + 6 + 2
            + (m + 1 + n))


def traffic_from_profiles(workload: str, io_bytes_per_launch: float):
    """HBM bytes per backward launch from the committed rocprofv3 PMC summary, or None when
    absent or taken on a different kernel source."""
    path = os.path.join(PROFILES, f"grkan_bwd_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def error_stats(got: np.ndarray, ref: np.ndarray) -> dict:
    e = got.astype(np.float64) - ref
    rel = np.abs(e) / np.maximum(np.abs(ref), 1e-300)
    return {"mae": float(np.mean(np.abs(e))), "var": float(np.var(e)), "max_rel": float(np.max(rel))}


def host_info() -> dict:
    """The host the CPU baseline ran on: logical CPUs, the ones this process may use, the CPU
    share declared through OMP_NUM_THREADS, and the CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count()
    return {"nproc": os.cpu_count(), "affinity": affinity,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "cpu_model": model}


def cpu_baseline(w, target_s: float = 10.0) -> dict:
    """The fp64 oracle, as it is, on the first rows of the workload: the forward alone (Y) and
    the forward + backward (Y, dX, dA, dB: the oracle evaluates each element's value and
    derivatives together), timed separately on the same rows, on the host's CPU share; and the
    same forward + backward on one thread on a smaller sample."""
    from gr_kan_rational_amd import synth
    from oracle import oracle

    def run(inp, with_dy, nthreads=None):
        t0 = time.perf_counter()
        oracle.run(inp["x"], inp["A"], inp["B"], w.n_groups, dy=inp["dy"] if with_dy else None, io=w.io,
                   m=w.m, n=w.n, nthreads=nthreads)
        return time.perf_counter() - t0

    calib_rows = min(256, w.rows)
    dt = run(synth.make_inputs(w, rows=calib_rows), True)
    rows = int(min(w.rows, max(calib_rows, calib_rows * target_s / max(dt, 1e-3))))
    inp = synth.make_inputs(w, rows=rows)
    run(inp, True)  # first touch of the output buffers' pages, outside the timing
    # a workload the oracle finishes in well under a second (tiny) is repeated until ~1 s
    reps = max(1, int(1.0 / max(run(inp, True), 1e-6))) if rows == w.rows else 1
    dt = sum(run(inp, True) for _ in range(reps)) / reps
    dt_fwd = sum(run(inp, False) for _ in range(reps)) / reps
    n = rows * w.d
    c1 = min(rows, calib_rows)
    rows1 = int(min(rows, max(c1, c1 * target_s / 4 / max(run(synth.make_inputs(w, rows=c1), True, 1), 1e-3))))
    inp1 = synth.make_inputs(w, rows=rows1)
    reps1 = max(1, int(0.5 / max(run(inp1, True, 1), 1e-6))) if rows1 == w.rows else 1
    dt1 = sum(run(inp1, True, 1) for _ in range(reps1)) / reps1
    return {"value": n / dt, "unit": "elements/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"first {rows} of {w.rows} rows ({n} elements) of {w.name}: forward + backward (Y, dX, dA, "
                      f"dB) in fp64, {dt:.3g} s wall (mean of {reps}); the forward alone (Y) on the same rows "
                      f"{dt_fwd:.3g} s",
            "forward_value": n / dt_fwd,
            "value_1_thread": rows1 * w.d / dt1,
            "sample_1_thread": f"first {rows1} rows ({rows1 * w.d} elements), forward + backward, {dt1:.1f} s wall",
            "host": host_info()}


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published


def cpu_baseline_layer(w, target_s: float = 10.0) -> dict:
    """fp64 layer oracle, forward (bf16(F(x)) W^T) and backward (dW, dx, dA, dB), on the
    first rows of the workload."""
    from gr_kan_rational_amd import synth
    from oracle import layer, oracle

    Wb = synth.weight(w)

    def run(rows):
        inp = synth.make_inputs(w, rows=rows)
        t0 = time.perf_counter()
        layer.forward(inp["x"], inp["A"], inp["B"], Wb, w.n_groups)
        layer.backward(inp["x"], inp["dz"], inp["A"], inp["B"], Wb, w.n_groups)
        return time.perf_counter() - t0

    calib = 64
    dt = run(calib)
    rows = int(min(w.rows, max(calib, calib * target_s / max(dt, 1e-3))))
    dt = run(rows)
    flops = 3 * 2.0 * rows * w.d * w.d_out
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"first {rows} of {w.rows} rows of {w.name}: forward and backward, F in fp64 with bf16 "
                      f"rounding, fp64 matrix products, {dt:.1f} s wall", "host": host_info()}


def bench_layer(args, w, gk, synth, dev, log) -> int:
    """The GR-KAN layer (bf16): a step is the forward z = F(x) W^T (grkan_layer_forward_ws: F
    fused into the matrix-core GEMM while z has one 256-column tile, else F once into a workspace
    and the plain GEMM) and the backward (grkan_layer_backward: dW, dx, dA, dB); three GEMMs of
    2 rows d_in d_out FLOPs each.  `detail` adds the fused form, the unfused composition through
    the public entry points (grkan_forward -> grkan_linear_forward) and, for context,
    grkan_forward followed by torch's library GEMM."""
    import torch

    log(f"layer workload {w.name}: x [{w.batch},{w.seq},{w.d}] -> {w.d_out}, bf16: generating inputs")
    inp = synth.make_inputs(w)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    x, W, dz = bf(inp["x"]), bf(inp["W"]), bf(inp["dz"])
    A = torch.from_numpy(inp["A"]).to(dev)
    B = torch.from_numpy(inp["B"]).to(dev)
    del inp
    z = torch.empty((w.rows, w.d_out), dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    dA = torch.empty((w.n_groups, 6), dtype=torch.float32, device=dev)
    dB = torch.empty((w.n_groups, 4), dtype=torch.float32, device=dev)
    dW = torch.empty((w.d_out, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(gk.grkan_layer_backward_workspace_size(w.rows, w.d, w.d_out, w.n_groups),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    fws_bytes = gk.grkan_layer_forward_workspace_size(w.rows, w.d, w.d_out, w.n_groups)
    fws = torch.empty(max(fws_bytes, 16), dtype=torch.uint8, device=dev)

    def forward():
        # the faster form for the shape (unfused beyond one 256-column tile of z)
        gk.grkan_layer_forward_ws(x, A, B, W, w.n_groups, out=z, workspace=fws, stream=stream)

    def fused():
        gk.grkan_layer_forward(x, A, B, W, w.n_groups, out=z, stream=stream)

    def backward():
        gk.grkan_layer_backward(x, dz, A, B, W, w.n_groups, dx=dx, dA=dA, dB=dB, dW=dW, workspace=ws,
                                stream=stream)

    def step():
        forward()
        backward()

    def unfused():
        gk.grkan_forward(x, A, B, w.n_groups, out=y, stream=stream)
        gk.grkan_linear_forward(y, W, out=z, stream=stream)

    def timed(fn, reps):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(reps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ms = timed(step, args.steps)
    gemm_flops = 2.0 * w.rows * w.d * w.d_out
    flops = 3 * gemm_flops
    tflops = flops / (ms * 1e-3) / 1e12
    fwd_ms = timed(forward, args.steps)
    bwd_ms = timed(backward, args.steps)
    detail = {
        "forward_ms": fwd_ms, "backward_ms": bwd_ms,
        "forward_form": "unfused (activation kernel, then the matrix product)" if fws_bytes else "fused",
        "fused_ms": timed(fused, args.steps),
        "forward_TFLOPs": gemm_flops / (fwd_ms * 1e-3) / 1e12,
        "backward_TFLOPs": 2 * gemm_flops / (bwd_ms * 1e-3) / 1e12,
        "unfused_ms": timed(unfused, args.steps),
        "activation_ms": timed(lambda: gk.grkan_forward(x, A, B, w.n_groups, out=y, stream=stream), args.steps),
        "linear_ms": timed(lambda: gk.grkan_linear_forward(y, W, out=z, stream=stream), args.steps),
        "torch_linear_ms": timed(lambda: torch.matmul(y, W.t(), out=z), args.steps),
        "flops_per_step": flops,
        "device": torch.cuda.get_device_name(dev),
    }
    detail["torch_unfused_ms"] = detail["activation_ms"] + detail["torch_linear_ms"]
    log(f"step {ms:.4f} ms ({tflops:.1f} TFLOP/s); forward ({detail['forward_form']}) {fwd_ms:.4f} ms, "
        f"fused {detail['fused_ms']:.4f} ms, backward {bwd_ms:.4f} ms; "
        f"unfused forward {detail['unfused_ms']:.4f} ms; "
        f"activation {detail['activation_ms']:.4f} + linear {detail['linear_ms']:.4f} ms; "
        f"torch linear {detail['torch_linear_ms']:.4f} ms")
    out = {
        "metric": f"GR-KAN layer forward + backward TFLOP/s (bf16 matrix cores), workload {w.name}",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 (fp32 accumulation)",
        "data": "synthetic",
        "config": {"workload": w.name, "shape": [w.batch, w.seq, w.d], "d_out": w.d_out,
                   "n_groups": w.n_groups, "degrees": [w.m, w.n], "io": "bf16"},
        "roofline": {"bound": "mfma", "achieved": detail["forward_TFLOPs"], "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": detail["forward_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "grkan_layer_forward_ws (" + detail["forward_form"] + ")",
                     "algorithmic_flops_per_launch": gemm_flops},
        "detail": detail,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 layer oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline_layer(w)
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline_cheby(w, target_s: float = 10.0) -> dict:
    """fp64 Chebyshev-KAN oracle, forward and backward, on the first rows of the workload."""
    from gr_kan_rational_amd import synth
    from oracle import chebykan, oracle

    C = synth.weight(w)

    def run(rows):
        inp = synth.make_inputs(w, rows=rows)
        t0 = time.perf_counter()
        chebykan.forward(inp["x"], C, w.cheby)
        chebykan.backward(inp["x"], inp["dz"], C, w.cheby)
        return time.perf_counter() - t0

    calib = 64
    dt = run(calib)
    rows = int(min(w.rows, max(calib, calib * target_s / max(dt, 1e-3))))
    dt = run(rows)
    flops = 3 * 2.0 * rows * w.d * (w.cheby + 1) * w.d_out
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"first {rows} of {w.rows} rows of {w.name}: forward and backward in fp64 (basis rounded "
                      f"to bf16), {dt:.1f} s wall", "host": host_info()}


def bench_cheby(args, w, gk, synth, dev, log) -> int:
    """The Chebyshev-KAN layer (bf16, degree 7): a step is the forward (basis built while
    staging the GEMM's A operand) and the backward (dC on the matrix cores with the basis built
    while staging, G = dy C, dx); three GEMMs of 2 rows 8 d_in d_out FLOPs each.  `detail`
    adds, for context, the same forward in eager torch ops (tanh, the recurrence in bf16 tensors,
    a library GEMM)."""
    import torch

    log(f"Chebyshev-KAN workload {w.name}: x [{w.batch},{w.seq},{w.d}] -> {w.d_out}, degree {w.cheby}")
    inp = synth.make_inputs(w)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    x, C, dy = bf(inp["x"]), bf(inp["W"]), bf(inp["dz"])
    del inp
    y = torch.empty((w.rows, w.d_out), dtype=torch.bfloat16, device=dev)
    dx = torch.empty_like(x)
    dC = torch.empty(C.shape, dtype=torch.float32, device=dev)
    ws = torch.empty(gk.grkan_chebykan_backward_workspace_size(w.rows, w.d, w.d_out, w.cheby),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def forward():
        gk.grkan_chebykan_forward(x, C, w.cheby, out=y, stream=stream)

    def backward():
        gk.grkan_chebykan_backward(x, dy, C, w.cheby, dx=dx, dC=dC, workspace=ws, stream=stream)

    def step():
        forward()
        backward()

    def timed(fn, reps):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(reps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ms = timed(step, args.steps)
    gemm_flops = 2.0 * w.rows * w.d * (w.cheby + 1) * w.d_out
    tflops = 3 * gemm_flops / (ms * 1e-3) / 1e12
    fwd_ms = timed(forward, args.steps)
    bwd_ms = timed(backward, args.steps)
    Cm = C.view(w.d_out, -1)

    def torch_forward():
        t = torch.tanh(x)
        T = [torch.ones_like(t), t]
        for _ in range(w.cheby - 1):
            T.append(2 * t * T[-1] - T[-2])
        return torch.matmul(torch.stack(T, dim=-1).view(w.rows, -1), Cm.t())

    detail = {"forward_ms": fwd_ms, "backward_ms": bwd_ms,
              "forward_TFLOPs": gemm_flops / (fwd_ms * 1e-3) / 1e12,
              "backward_TFLOPs": 2 * gemm_flops / (bwd_ms * 1e-3) / 1e12,
              "torch_eager_forward_ms": timed(torch_forward, max(3, args.steps // 5)),
              "flops_per_step": 3 * gemm_flops, "device": torch.cuda.get_device_name(dev)}
    log(f"step {ms:.4f} ms ({tflops:.1f} TFLOP/s); forward {fwd_ms:.4f} ms, backward {bwd_ms:.4f} ms; "
        f"torch eager forward {detail['torch_eager_forward_ms']:.4f} ms")
    out = {
        "metric": f"Chebyshev-KAN layer forward + backward TFLOP/s (bf16 matrix cores, basis built in the GEMM "
                  f"staging), workload {w.name}",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 (fp32 accumulation)", "data": "synthetic",
        "config": {"workload": w.name, "shape": [w.batch, w.seq, w.d], "d_out": w.d_out, "degree": w.cheby,
                   "io": "bf16"},
        "roofline": {"bound": "mfma", "achieved": detail["forward_TFLOPs"], "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": detail["forward_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "grkan_chebykan_forward (grkan_layer_gemm_kernel, Chebyshev prologue)",
                     "algorithmic_flops_per_launch": gemm_flops},
        "detail": detail,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 Chebyshev-KAN oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline_cheby(w)
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="kat-b")
    ap.add_argument("--mode", choices=["deterministic", "block_atomic"], default="deterministic")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-naive", action="store_true")
    ap.add_argument("--inflate", default="2,4,8",
                    help="repeat counts of the FLOP-inflation probe timed after the step (GR-KAN "
                         "degrees only; 'none' to skip)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of one workload tensor (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the activation would shard by rows, with no "
              "communication but an all-reduce of dA/dB, and no multi-GPU path is implemented; "
              "use --gpus 1", file=sys.stderr)
        return 2

    import torch

    import gr_kan_rational_amd.binding as gk
    from gr_kan_rational_amd import synth

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    if args.copy_probe:
        # A plain copy of known size: what FETCH_SIZE / WRITE_SIZE read for it calibrates the
        # counters that measure the GR-KAN kernels' HBM traffic.
        nbytes = w.elements * w.io_bytes
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes,
                          "copies": max(1, args.steps)}), flush=True)
        return 0
    gk.load_library()
    if w.cheby:
        return bench_cheby(args, w, gk, synth, dev, log)
    if w.d_out > 0:
        return bench_layer(args, w, gk, synth, dev, log)
    io = gk.GRKAN_BF16 if w.io == "bf16" else gk.GRKAN_F32
    log(f"workload {w.name} [{w.batch},{w.seq},{w.d}] {w.io}: generating inputs")
    inp = synth.make_inputs(w)

    def to_dev(a):
        if w.io == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    x, dy = to_dev(inp["x"]), to_dev(inp["dy"])
    A = torch.from_numpy(inp["A"]).to(dev)
    B = torch.from_numpy(inp["B"]).to(dev) if w.n > 0 else None
    del inp
    E = w.elements
    es = w.io_bytes
    # Input sets, rotated call by call so that no call finds its operands in the 256 MB Infinity
    # Cache (MALL) from the call before: one set when a set (x, dy, y, dx) is already far larger
    # than that cache (KAT-B: 2.5 GB), else copies of the same inputs in distinct buffers until
    # the sets together hold MALL_DEFEAT_BYTES (KAT-T: 28 sets of 77 MB).
    set_bytes = 4 * E * es
    n_sets = int(min(MAX_SETS, max(1, -(-MALL_DEFEAT_BYTES // set_bytes))))
    sets = [(x, dy, torch.empty_like(x), torch.empty_like(x))]
    for _ in range(n_sets - 1):
        sets.append((x.clone(), dy.clone(), torch.empty_like(x), torch.empty_like(x)))
    dA = torch.empty((w.n_groups, w.m + 1), dtype=torch.float32, device=dev)
    dB = torch.empty((w.n_groups, w.n), dtype=torch.float32, device=dev) if w.n > 0 else None
    # GR-KAN itself (degrees (5, 4)) goes through the grkan_* entry points, the other
    # members of the PAU family through grkan_pau_*.
    pau = (w.m, w.n) != (5, 4)
    if pau:
        ws_bytes = gk.grkan_pau_backward_workspace_size(w.rows, w.d, w.n_groups, w.m, w.n, io, 0)
    else:
        ws_bytes = gk.grkan_backward_workspace_size(w.rows, w.d, w.n_groups, io, 0)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def fwd(i=0):
        xs, _, ys, _ = sets[i % n_sets]
        if pau:
            gk.grkan_pau_forward(xs, A, B, w.n_groups, w.m, w.n, out=ys, stream=stream)
        else:
            gk.grkan_forward(xs, A, B, w.n_groups, out=ys, stream=stream)

    def bwd(i=0, mode=args.mode):
        xs, dys, _, dxs = sets[i % n_sets]
        if pau:
            gk.grkan_pau_backward(xs, dys, A, B, w.n_groups, w.m, w.n, mode=mode,
                                  dx=dxs, dA=dA, dB=dB, workspace=ws, stream=stream)
        else:
            gk.grkan_backward(xs, dys, A, B, w.n_groups, mode=mode,
                              dx=dxs, dA=dA, dB=dB, workspace=ws, stream=stream)

    def probe(i=0):
        xs, dys, _, dxs = sets[i % n_sets]
        gk.grkan_stream_probe(xs, dys, out=dxs, stream=stream)

    def launch(pass_):
        if pau:
            return gk.grkan_pau_query_launch(w.rows, w.d, w.n_groups, w.m, w.n, io, pass_)
        return gk.grkan_query_launch(w.rows, w.d, w.n_groups, io, pass_)

    def step(i=0):
        fwd(i)
        bwd(i)

    log(f"warmup {args.warmup} steps ({n_sets} input set(s) of {set_bytes / 1e6:.1f} MB)")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def timed(fn, reps):
        """Average duration (ms) of fn over reps back-to-back calls (rotating the input sets),
        bracketed by two HIP events on the stream the kernels run on."""
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        fn(0)  # first call outside the timing (loads the code object if not yet loaded)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(reps):
            fn(i + 1)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_sum = torch.empty((), dtype=torch.float32, device=dev)

    def timed_flushed(fn, reps):
        """Average duration (ms) of fn with the Infinity Cache flushed before each call (a read of
        FLUSH_BYTES outside the events; a read leaves clean lines, so the call pays no write-back
        of the flush itself): a cross-check of the rotation."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i, (e0, e1) in enumerate(ev):
            torch.sum(flush, dim=0, out=flush_sum)
            e0.record(stream)
            fn(i)
            e1.record(stream)
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in ev) / reps

    log(f"timing {args.steps} steps")
    wall0 = time.perf_counter()
    ms_per_step = timed(step, args.steps)
    wall = time.perf_counter() - wall0
    # Per-kernel averages for the roofline: the same calls, timed in their own back-to-back loops.
    bwd_ms = timed(bwd, args.steps)
    fwd_ms = timed(fwd, args.steps)
    # The measured ceiling of the backward's traffic (two tensors read, one written) on this
    # device: the library's streaming probe over the same buffers.
    probe_ms = timed(probe, args.steps)
    bwd_ms_flushed = timed_flushed(bwd, min(args.steps, 20))
    fwd_ms_flushed = timed_flushed(fwd, min(args.steps, 20))
    del flush, flush_sum
    value = E / (ms_per_step * 1e-3)
    bwd_bytes = 3 * es * E
    fwd_bytes = 2 * es * E
    bwd_gbps = bwd_bytes / (bwd_ms * 1e-3) / 1e9
    fwd_gbps = fwd_bytes / (fwd_ms * 1e-3) / 1e9
    probe_gbps = bwd_bytes / (probe_ms * 1e-3) / 1e9
    log(f"step {ms_per_step:.4f} ms; fwd {fwd_ms:.4f} ms, bwd {bwd_ms:.4f} ms ({bwd_gbps:.0f} GB/s); "
        f"stream probe {probe_ms:.4f} ms ({probe_gbps:.0f} GB/s); flushed fwd {fwd_ms_flushed:.4f} / "
        f"bwd {bwd_ms_flushed:.4f} ms; wall {wall:.3f} s")

    detail = {
        "elements": E,
        "input_sets": n_sets, "input_set_bytes": set_bytes,
        "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
        "fwd_GBps": fwd_gbps, "fwd_frac_hbm_peak": fwd_gbps / HBM_PEAK_GBPS,
        "bwd_GBps": bwd_gbps, "bwd_frac_hbm_peak": bwd_gbps / HBM_PEAK_GBPS,
        "fwdbwd_GBps": (fwd_bytes + bwd_bytes) / (ms_per_step * 1e-3) / 1e9,
        "fwd_ms_flushed": fwd_ms_flushed, "bwd_ms_flushed": bwd_ms_flushed,
        "stream_probe_ms": probe_ms, "stream_probe_GBps": probe_gbps,
        "bwd_frac_of_stream_probe": probe_ms / bwd_ms,
        "launch_fwd": launch(0),
        "launch_bwd": launch(1),
        "device": torch.cuda.get_device_name(dev),
    }
    # the rest uses the first set only
    x, dy, y, dx = sets[0]
    sets = sets[:1]
    n_sets = 1
    torch.cuda.empty_cache()

    # other backward modes, outside the timed region
    def time_one(fn, reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        s.record(stream)
        for _ in range(reps):
            fn()
        e.record(stream)
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    golden = os.path.join(GOLDEN, f"{w.name}.sums.json")
    ref = None
    if os.path.exists(golden):
        with open(golden) as f:
            g = json.load(f)
        ref = (np.array(g["dA"]), np.array(g["dB"]))
    errors = {}

    def grad_errors():
        e = {"dA": error_stats(dA.cpu().numpy(), ref[0])}
        if dB is not None:
            e["dB"] = error_stats(dB.cpu().numpy(), ref[1])
        return e

    other = "block_atomic" if args.mode == "deterministic" else "deterministic"
    detail[f"bwd_{other}_ms"] = time_one(lambda: bwd(0, other), 10)
    for mode in ("deterministic", "block_atomic"):
        bwd(0, mode)
        torch.cuda.synchronize()
        if ref is not None:
            errors[mode] = grad_errors()
    if not args.no_naive and not pau:
        log("naive per-element-atomic backward (one run)")
        detail["bwd_naive_ms"] = time_one(lambda: bwd(0, "naive"), 1)
        if ref is not None:
            errors["naive_per_element_atomic"] = grad_errors()
    if errors:
        detail["grad_error_vs_fp64_oracle"] = errors

    repeats = [] if args.inflate == "none" or pau else [int(r) for r in args.inflate.split(",")]
    if repeats and w.d % w.n_groups == 0 and (w.d // w.n_groups * es) % 16 == 0:
        # The pages' Insight 2: the same calls with each element's arithmetic repeated R times
        # (outputs unchanged).  Flat times mean the arithmetic is hidden under the memory
        # stream; times growing with R mean the kernel is near or past the point where its
        # arithmetic, not HBM, sets the pace.
        log(f"FLOP-inflation probe, repeats {repeats}")
        infl = {"repeats": [1], "fwd_ms": [fwd_ms], "bwd_ms": [bwd_ms]}
        for r in repeats:
            infl["repeats"].append(r)
            infl["fwd_ms"].append(time_one(
                lambda: gk.grkan_inflated_forward(x, A, B, w.n_groups, repeat=r, out=y, stream=stream),
                args.steps))
            infl["bwd_ms"].append(time_one(
                lambda: gk.grkan_inflated_backward(x, dy, A, B, w.n_groups, repeat=r, dx=dx, dA=dA,
                                                   dB=dB, workspace=ws, stream=stream), args.steps))
        infl["fwd_vs_plain"] = [t / fwd_ms for t in infl["fwd_ms"]]
        infl["bwd_vs_plain"] = [t / bwd_ms for t in infl["bwd_ms"]]
        detail["flop_inflation"] = infl

    traffic = traffic_from_profiles(w.name, bwd_bytes)
    out = {
        "metric": ("GR-KAN fwd+bwd elements/s and achieved HBM GB/s (% peak) at KAT-B shape"
                   if w.name == "kat-b" else
                   f"GR-KAN/PAU fwd+bwd elements/s and achieved HBM GB/s (% peak), workload {w.name}"),
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.io == "f32" else "f32 (bf16 I/O)",
        "data": "synthetic",
        "config": {"workload": w.name, "shape": [w.batch, w.seq, w.d], "n_groups": w.n_groups,
                   "degrees": [w.m, w.n], "io": w.io, "backward_mode": args.mode},
        "roofline": {"bound": "hbm", "achieved": bwd_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": bwd_gbps / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": ("grkan_pau_backward" if pau else "grkan_backward")
                               + " (main kernel + fixed-order merge)",
                     "algorithmic_bytes_per_launch": bwd_bytes},
        "detail": detail,
    }
    if w.io == "bf16" and w.n > 0 and w.m > 0:
        # bf16 I/O halves the bytes per element but not the arithmetic: this backward is bound
        # by its vector-ALU work, and is rated against the vector-ALU issue peak instead (its
        # HBM figures stay under detail)
        ops = backward_valu_ops_per_element(w.m, w.n, w.io)
        tops = ops * E / (bwd_ms * 1e-3) / 1e12
        out["roofline"] = {"bound": "alu", "achieved": tops, "peak": VALU_PEAK_TOPS, "unit": "TOP/s",
                           "frac": tops / VALU_PEAK_TOPS, "traffic": traffic,
                           "kernel": out["roofline"]["kernel"], "valu_ops_per_element": ops,
                           "elements_per_launch": E,
                           "hbm": {"achieved": bwd_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                   "frac": bwd_gbps / HBM_PEAK_GBPS, "algorithmic_bytes_per_launch": bwd_bytes}}
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
