"""Benchmark: Gaussian kernel sum pair evaluations per second on one MI355X.

One step is one call of keops_gauss_sum on inputs already resident in HBM: the operand
preparation (bounds, row and column pieces) plus the fused reduction kernel over all M x N pairs
and the combine of the column splits. The default workload is the
1M x 1M, D=3, C=1, float32, sigma=0.01 Gauss sum. Timing uses HIP events recorded on the
stream the kernels run on, after W warm-up steps, bracketed by device synchronisations.

Prints ONE JSON line (the contract), with extra objects:
  step_stats    per-step times: mean +- 1 std (sample), median, min, max
  roofline      the dominant kernel against the float32 vector peak (ALU-bound)
  cpu_baseline  the float64 CPU oracle on a bounded row sample of the same workload
  secondary     the batched fp16 Gauss sum (B=4, M=N=16384, D=C=32) on the matrix cores, timed
                over at least 100 calls, with its forward sweep against the fp16 matrix-core peak
--all additionally times the other workloads and writes them to --all-out (not the line).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Peaks (MI355X, 256 CUs at 2.4 GHz). Float32 vector: 256 CU x 4 SIMD x 16 lanes x 2 flop
# (FMA) x 2 (packed dual-issue) x 2.4 GHz = 157.3 TFLOP/s. Dense fp16 matrix: 2516.6 TFLOP/s.
PEAK_FP32_VECTOR_TFLOPS = 157.3
PEAK_FP16_MFMA_TFLOPS = 2516.6
# Algorithmic work per pair (fixed convention): Gauss sum 3D + 1 + 2C flop (12 at D=3, C=1);
# gradient 5D + 2C + 1; matrix-core path 2(D + C).
def gauss_flops_per_pair(D, C):
    return 3 * D + 1 + 2 * C


def grad_flops_per_pair(D, C):
    return 5 * D + 2 * C + 1


# HBM bytes per launch of the dominant kernel on the 1M workload, from rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE (each scaled by what it reads for a 256 MiB copy: x2.0 and x1.0).
# Reported only while the sources the kernel is compiled from are byte-identical to the ones
# that were measured (sha256 over the listed files, concatenated in order).
MEASURED_TRAFFIC = {"bytes": 2189558713,
                    "sources": ["pairwise_reductions_amd/csrc/lowd_mfma.hip",
                                "pairwise_reductions_amd/csrc/lowd_common.h",
                                "pairwise_reductions_amd/csrc/lowd.hip"],
                    "sha256_prefix": "94fdaf6b8e4b2c1e"}


def kernel_source_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    if not MEASURED_TRAFFIC["bytes"] or not MEASURED_TRAFFIC["sha256_prefix"]:
        return None
    try:
        digest = kernel_source_digest(MEASURED_TRAFFIC["sources"])
    except OSError:
        return None
    return MEASURED_TRAFFIC["bytes"] if digest.startswith(MEASURED_TRAFFIC["sha256_prefix"]) else None


def _events_time(fn, steps, warmup, before_timed=None, per_step=None):
    """Seconds per step over `steps` timed steps after `warmup` untimed ones, from HIP events on
    the current stream. With a list `per_step`, an event is recorded between consecutive steps
    as well and the list receives every step's own duration in milliseconds."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if before_timed is not None:
        before_timed()
    stream = torch.cuda.current_stream()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1 if per_step is not None else 2)]
    marks[0].record(stream)
    for k in range(steps):
        fn()
        if per_step is not None:
            marks[k + 1].record(stream)
    marks[-1].record(stream)
    torch.cuda.synchronize()
    if per_step is not None:
        per_step.extend(marks[k].elapsed_time(marks[k + 1]) for k in range(steps))
    return marks[0].elapsed_time(marks[-1]) / 1e3 / steps  # seconds per step


def _stats(ms):
    """mean +- 1 std (sample), median, min and max of per-step milliseconds."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"reps": int(a.size), "mean_ms": float(a.mean()), "std_ms": float(a.std(ddof=1)) if a.size > 1 else 0.0,
            "median_ms": float(np.median(a)), "min_ms": float(a.min()), "max_ms": float(a.max())}


def bench_gauss_1m(steps, warmup, cpu_rows, cpu_baseline=True):
    import numpy as np
    import torch

    import pairwise_reductions_amd as pr
    from pairwise_reductions_amd import _lib, workloads

    key = "gauss_sum_1m"
    inp = workloads.make_inputs(key)
    M, N, D, C = inp["M"], inp["N"], inp["D"], inp["C"]
    sigma = float(inp["sigma"])
    dev = torch.device("cuda:0")
    x, y, b = (torch.from_numpy(inp[k]).to(dev) for k in ("x", "y", "b"))
    out = torch.empty((M, C), dtype=torch.float32, device=dev)
    nbytes = pr.workspace_bytes(_lib.OP_GAUSS_SUM, 1, M, N, D, C, 0, _lib.KEOPS_F32)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        pr.gauss_sum(x, y, b, sigma, out=out, workspace=ws)

    # The step (every kernel of the call) is timed with events on the current stream; the
    # library also records an event pair on that stream around each launch of the dominant
    # kernel, the matrix-core sweep, which gives that kernel's own average duration.
    lib = _lib.load()
    per_step = []
    t = _events_time(step, steps, warmup, before_timed=lambda: _lib.check(lib.keops_sweep_timing(1),
                                                                           "keops_sweep_timing"),
                     per_step=per_step)
    sweep_ms, sweeps = ctypes.c_float(0.0), ctypes.c_int(0)
    _lib.check(lib.keops_sweep_timing_read(ctypes.byref(sweep_ms), ctypes.byref(sweeps)), "keops_sweep_timing_read")
    _lib.check(lib.keops_sweep_timing(0), "keops_sweep_timing")
    kernel_s = sweep_ms.value / 1e3 / sweeps.value if sweeps.value == steps else t
    pairs = float(M) * float(N)
    flops = pairs * gauss_flops_per_pair(D, C)
    achieved = flops / kernel_s / 1e12
    result = {
        "metric": "Gauss-sum pair evals/s (M*N/s) at 1M x 1M, D=3, fp32",
        "value": pairs / t,
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": t * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: x, y uniform on the 2^-24 grid in [0,1)^3, b ~ N(0,1), seed 0",
        "config": {"workload": key, "M": M, "N": N, "D": D, "C": C, "sigma": sigma,
                   "pairs_per_step": pairs},
        "step_stats": _stats(per_step),
        "roofline": {
            "bound": "alu",
            "achieved": achieved,
            "peak": PEAK_FP32_VECTOR_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_VECTOR_TFLOPS,
            "traffic": measured_traffic(),
            "traffic_unit": "bytes per launch",
            "kernel": "gauss_sum_mf32_kernel<2>",
            "flop_per_pair": gauss_flops_per_pair(D, C),
            "kernel_ms": kernel_s * 1e3,
            "kernel_timing": "events around each launch" if sweeps.value == steps else "whole step",
        },
    }
    if cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_gauss(inp, cpu_rows)
    out_host = out.cpu().numpy()
    result["config"]["checksum"] = float(np.sum(out_host, dtype=np.float64))
    return result


def bench_fp16_secondary(reps, warmup):
    """The batched fp16 Gauss sum (B=4, M=N=16384, D=C=32, tau=1) on the matrix cores, as one
    extra object of the JSON line: whole-call time per rep (mean +- std, median) and the
    forward sweep's own average duration from events around each of its launches, against the
    dense fp16 matrix-core peak (2(D + C) flop per pair)."""
    import torch

    import pairwise_reductions_amd as pr
    from pairwise_reductions_amd import _lib, workloads

    key = "batched_gauss_sum_fp16"
    inp = workloads.make_inputs(key)
    Bt, M, N, D, C = inp["B"], inp["M"], inp["N"], inp["D"], inp["C"]
    dev = torch.device("cuda:0")
    q, k, v = _resident(inp, ("x", "y", "b"), dev)
    sig = float(inp["sigma"])
    out = torch.empty((Bt, M, C), device=dev)
    ws = torch.empty(max(1, pr.workspace_bytes(_lib.OP_GAUSS_SUM, Bt, M, N, D, C, 0, _lib.KEOPS_F16)),
                     dtype=torch.uint8, device=dev)
    lib = _lib.load()
    per_step = []
    t = _events_time(lambda: pr.gauss_sum(q, k, v, sig, out=out, workspace=ws), reps, warmup,
                     before_timed=lambda: _lib.check(lib.keops_sweep_timing(1), "keops_sweep_timing"),
                     per_step=per_step)
    sweep_ms, sweeps = ctypes.c_float(0.0), ctypes.c_int(0)
    _lib.check(lib.keops_sweep_timing_read(ctypes.byref(sweep_ms), ctypes.byref(sweeps)), "keops_sweep_timing_read")
    _lib.check(lib.keops_sweep_timing(0), "keops_sweep_timing")
    kernel_s = sweep_ms.value / 1e3 / sweeps.value if sweeps.value == reps else t
    pairs = float(Bt) * M * N
    mflops = pairs * 2 * (D + C)
    return {
        "workload": key, "B": Bt, "M": M, "N": N, "D": D, "C": C, "dtype": "f16", "tau": 1.0 / sig ** 2,
        "pairs_per_s": pairs / t, "ms_per_call": t * 1e3, "step_stats": _stats(per_step),
        "roofline": {"bound": "mfma", "achieved": mflops / kernel_s / 1e12, "peak": PEAK_FP16_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": mflops / kernel_s / 1e12 / PEAK_FP16_MFMA_TFLOPS,
                     "kernel": "fwd32_kernel<_Float16,4,128,8>", "flop_per_pair": 2 * (D + C),
                     "kernel_ms": kernel_s * 1e3,
                     "kernel_timing": "events around each launch" if sweeps.value == reps else "whole call",
                     "call_frac": mflops / t / 1e12 / PEAK_FP16_MFMA_TFLOPS},
    }


def cpu_baseline_gauss(inp, rows):
    import numpy as np

    import oracle
    from pairwise_reductions_amd import workloads

    workers = os.cpu_count() or 1
    sel = workloads.sample_rows(inp["M"], rows, seed=1, edge=0)
    xs = inp["x"][sel]
    t0 = time.perf_counter()
    oracle.gauss_sum(xs, inp["y"], inp["b"], float(inp["sigma"]), workers=workers)
    dt = time.perf_counter() - t0
    pairs = float(len(sel)) * float(inp["N"])
    return {"value": pairs / dt, "unit": "pairs/s", "cores": workers, "kind": "oracle",
            "sample": f"{len(sel)} seeded rows x all {inp['N']} columns ({pairs:.3g} pairs, {dt:.1f} s)",
            "seconds": dt}


def _oracle_rate(fn, pairs, sample):
    """The CPU oracle's rate on a bounded sample of a workload (timed beside the device figure)."""
    t0 = time.perf_counter()
    fn()
    dt = time.perf_counter() - t0
    return {"oracle_pairs_per_s": pairs / dt, "oracle_sample": f"{sample} ({pairs:.3g} pairs, {dt:.2f} s)",
            "oracle_cores": os.cpu_count() or 1}


def _resident(inp, keys, dev):
    import torch
    return [torch.from_numpy(inp[k]).to(dev) for k in keys]


ALL_GROUPS = ("gauss_sum_10k", "grad_100k", "fp16", "fp16_fwd_bwd", "fp16_d_sweep", "bf16_f32", "diffusion",
              "argkmin_lse", "gauss_sum_1m_outliers")


def bench_all(steps, warmup, only=None, cpu=True):
    """Time every workload through the library (inputs resident on the GPU); `only` names one
    group of ALL_GROUPS. With `cpu`, each group also reports the CPU oracle's rate on a bounded
    row sample of the same inputs (a few seconds each)."""
    import numpy as np
    import torch

    import pairwise_reductions_amd as pr
    from pairwise_reductions_amd import _lib, workloads

    dev = torch.device("cuda:0")
    rows = {}

    def want(group):
        return only is None or only == group

    # Gauss sum 10k (small case: launch-dominated)
    if want("gauss_sum_10k"):
        inp = workloads.make_inputs("gauss_sum_10k")
        x, y, b = _resident(inp, ("x", "y", "b"), dev)
        sig = float(inp["sigma"])
        out = torch.empty((inp["M"], inp["C"]), device=dev)
        ws = torch.empty(max(1, pr.workspace_bytes(0, 1, inp["M"], inp["N"], 3, 1)), dtype=torch.uint8, device=dev)
        t = _events_time(lambda: pr.gauss_sum(x, y, b, sig, out=out, workspace=ws), max(steps, 100), warmup)
        pairs = float(inp["M"]) * inp["N"]
        rows["gauss_sum_10k"] = {"ms": t * 1e3, "pairs_per_s": pairs / t,
                                 "frac_fp32_peak": pairs * 12 / t / 1e12 / PEAK_FP32_VECTOR_TFLOPS}
        if cpu:
            import oracle
            rows["gauss_sum_10k"].update(_oracle_rate(
                lambda: oracle.gauss_sum(inp["x"], inp["y"], inp["b"], sig, workers=os.cpu_count()),
                pairs, "all rows x all columns"))

    # Gauss sum forward + gradient of sum_i s_i^2 (g = 2 s), 100k mixture
    if want("grad_100k"):
        inp = workloads.make_inputs("gauss_sum_grad_x_100k_mixture")
        x, y, b = _resident(inp, ("x", "y", "b"), dev)
        sig = float(inp["sigma"])
        M, N = inp["M"], inp["N"]
        out = torch.empty((M, 1), device=dev)
        g = torch.empty((M, 1), device=dev)
        grad = torch.empty((M, 3), device=dev)
        ws = torch.empty(max(pr.workspace_bytes(0, 1, M, N, 3, 1), pr.workspace_bytes(3, 1, M, N, 3, 1), 1),
                         dtype=torch.uint8, device=dev)

        def fwd_bwd():
            pr.gauss_sum(x, y, b, sig, out=out, workspace=ws)
            torch.mul(out, 2.0, out=g)
            pr.gauss_sum_grad_x(x, y, b, g, sig, out=grad, workspace=ws)

        t = _events_time(fwd_bwd, steps, warmup)
        tf = _events_time(lambda: pr.gauss_sum(x, y, b, sig, out=out, workspace=ws), steps, warmup)
        tb = _events_time(lambda: pr.gauss_sum_grad_x(x, y, b, g, sig, out=grad, workspace=ws), steps, warmup)
        pairs = float(M) * N
        rows["gauss_sum_grad_x_100k_mixture"] = {
            "ms": t * 1e3, "fwd_ms": tf * 1e3, "grad_ms": tb * 1e3, "pairs_per_s": 2 * pairs / t,
            "frac_fp32_peak": pairs * (12 + grad_flops_per_pair(3, 1)) / t / 1e12 / PEAK_FP32_VECTOR_TFLOPS}
        if cpu:
            import oracle
            n = 1024
            gs = workloads.upstream_gradient(n, 1, seed=2)

            def oracle_fwd_bwd():
                oracle.gauss_sum(inp["x"][:n], inp["y"], inp["b"], sig, workers=os.cpu_count())
                oracle.gauss_sum_grad_x(inp["x"][:n], inp["y"], inp["b"], gs, sig, workers=os.cpu_count())

            rows["gauss_sum_grad_x_100k_mixture"].update(_oracle_rate(
                oracle_fwd_bwd, 2.0 * n * N, f"forward + gradient, first {n} rows x all {N} columns"))

    # Batched Gauss sum, fp16 matrix-core path: B=4, M=N=16384, D=C=32, tau=1
    if want("fp16"):
        inp = workloads.make_inputs("batched_gauss_sum_fp16")
        q, k, v = _resident(inp, ("x", "y", "b"), dev)
        Bt, M, N, D, C = inp["B"], inp["M"], inp["N"], inp["D"], inp["C"]
        out = torch.empty((Bt, M, C), device=dev)
        ws = torch.empty(max(1, pr.workspace_bytes(0, Bt, M, N, D, C, 0, _lib.KEOPS_F16)), dtype=torch.uint8,
                         device=dev)
        t = _events_time(lambda: pr.gauss_sum(q, k, v, float(inp["sigma"]), out=out, workspace=ws),
                         max(steps, 100), warmup)
        pairs = float(Bt) * M * N
        mflops = pairs * 2 * (D + C)
        rows["batched_gauss_sum_fp16"] = {"ms": t * 1e3, "pairs_per_s": pairs / t,
                                          "mfma_tflops": mflops / t / 1e12,
                                          "frac_fp16_mfma_peak": mflops / t / 1e12 / PEAK_FP16_MFMA_TFLOPS}
        if cpu:
            import oracle
            n = 256
            rows["batched_gauss_sum_fp16"].update(_oracle_rate(
                lambda: oracle.gauss_sum_batched(inp["x"][:, :n], inp["y"], inp["b"], 1.0 / float(inp["sigma"]) ** 2,
                                                 workers=os.cpu_count()),
                float(Bt) * n * N, f"first {n} rows of each of the {Bt} problems x all {N} columns"))

    # Batched Gauss sum forward + backward, fp16: B=4, M=N=16384, D=32, C=1 (the flash page's
    # Figure 2 shape); the backward computes the gradients with respect to x, y and b.
    if want("fp16_fwd_bwd"):
        inp = workloads.make_inputs("batched_gauss_sum_fp16_fwd_bwd")
        q, k, v = _resident(inp, ("x", "y", "b"), dev)
        Bt, M, N, D, C = inp["B"], inp["M"], inp["N"], inp["D"], inp["C"]
        sig = float(inp["sigma"])
        out = torch.empty((Bt, M, C), device=dev)
        gup = torch.from_numpy(workloads.upstream_gradient(M, C, seed=4, B=Bt)).to(dev)
        ws = torch.empty(max(1, pr.workspace_bytes(_lib.OP_GAUSS_SUM_BACKWARD, Bt, M, N, D, C, 0, _lib.KEOPS_F16),
                             pr.workspace_bytes(0, Bt, M, N, D, C, 0, _lib.KEOPS_F16)), dtype=torch.uint8, device=dev)
        tf = _events_time(lambda: pr.gauss_sum(q, k, v, sig, out=out, workspace=ws), max(steps, 50), warmup)
        tb = _events_time(lambda: pr.gauss_sum_backward(q, k, v, gup, sig, workspace=ws), max(steps, 50), warmup)
        tbx = _events_time(lambda: pr.gauss_sum_backward(q, k, v, gup, sig, need=("x",), workspace=ws),
                           max(steps, 50), warmup)
        pairs = float(Bt) * M * N
        rows["batched_gauss_sum_fp16_fwd_bwd"] = {"fwd_ms": tf * 1e3, "bwd_ms": tb * 1e3, "bwd_x_only_ms": tbx * 1e3,
                                                  "fwd_bwd_ms": (tf + tb) * 1e3, "fwd_pairs_per_s": pairs / tf}

    # Sweep over D of the fp16 forward at B=64, M=N=16384, C=1 (the flash page's Figure 3 shape)
    if want("fp16_d_sweep"):
        for D in (16, 32, 64, 128):
            Bt, M, N, C = 64, 16384, 16384, 1
            rng = torch.Generator(device="cpu").manual_seed(D)
            q = (torch.randn((Bt, M, D), generator=rng) / D ** 0.5).to(torch.float16).to(dev)
            k = (torch.randn((Bt, N, D), generator=rng) / D ** 0.5).to(torch.float16).to(dev)
            v = torch.randn((Bt, N, C), generator=rng).to(torch.float16).to(dev)
            out = torch.empty((Bt, M, C), device=dev)
            ws = torch.empty(max(1, pr.workspace_bytes(0, Bt, M, N, D, C, 0, _lib.KEOPS_F16)), dtype=torch.uint8,
                             device=dev)
            t = _events_time(lambda: pr.gauss_sum(q, k, v, 1.0, out=out, workspace=ws), max(steps, 20), warmup)
            pairs = float(Bt) * M * N
            rows[f"fp16_d_sweep_B64_C1_D{D}"] = {"ms": t * 1e3, "pairs_per_s": pairs / t}
            del q, k, v, out, ws

    # bf16 and float32 inputs on the matrix cores at the flash page's Figure 5 shape (B=4,
    # M=N=16384, D=C=32; float32 runs as fp16 hi + lo parts, three products each) and the
    # float32 D sweep of its Figure 4 shape (B=64, M=N=16384, C=1).
    if want("bf16_f32"):
        for dtype, name in ((torch.bfloat16, "bf16"), (torch.float32, "f32")):
            Bt, M, N, D, C = 4, 16384, 16384, 32, 32
            rng = torch.Generator(device="cpu").manual_seed(11)
            q = (torch.randn((Bt, M, D), generator=rng) / D ** 0.5).to(dtype).to(dev)
            k = (torch.randn((Bt, N, D), generator=rng) / D ** 0.5).to(dtype).to(dev)
            v = torch.randn((Bt, N, C), generator=rng).to(dtype).to(dev)
            out = torch.empty((Bt, M, C), device=dev)
            dt = _lib.KEOPS_BF16 if dtype == torch.bfloat16 else _lib.KEOPS_F32
            ws = torch.empty(max(1, pr.workspace_bytes(0, Bt, M, N, D, C, 0, dt)), dtype=torch.uint8, device=dev)
            t = _events_time(lambda: pr.gauss_sum(q, k, v, 1.0, out=out, workspace=ws), max(steps, 20), warmup)
            pairs = float(Bt) * M * N
            rows[f"batched_gauss_sum_{name}_B4_D32_C32"] = {"ms": t * 1e3, "pairs_per_s": pairs / t}
        for D in (16, 32, 64, 128):
            Bt, M, N, C = 64, 16384, 16384, 1
            rng = torch.Generator(device="cpu").manual_seed(D + 100)
            q = (torch.randn((Bt, M, D), generator=rng) / D ** 0.5).to(dev)
            k = (torch.randn((Bt, N, D), generator=rng) / D ** 0.5).to(dev)
            v = torch.randn((Bt, N, C), generator=rng).to(dev)
            out = torch.empty((Bt, M, C), device=dev)
            ws = torch.empty(max(1, pr.workspace_bytes(0, Bt, M, N, D, C, 0, _lib.KEOPS_F32)), dtype=torch.uint8,
                             device=dev)
            t = _events_time(lambda: pr.gauss_sum(q, k, v, 1.0, out=out, workspace=ws), max(steps, 5), warmup)
            rows[f"f32_d_sweep_B64_C1_D{D}"] = {"ms": t * 1e3, "pairs_per_s": float(Bt) * M * N / t}
            del q, k, v, out, ws

    # Diffusion operator (fp32, D=3): the q and d normalisation passes and one application of
    # diag(s) K diag(s) to a block of 4 vectors, N = 2^17.
    if want("diffusion"):
        N, D, Cb = 1 << 17, 3, 4
        rng = torch.Generator(device="cpu").manual_seed(7)
        xs = torch.rand((N, D), generator=rng).to(dev)
        vb = torch.randn((N, Cb), generator=rng).to(dev)
        sv, qv, dv = pr.diffusion_scaling(xs, 0.05, 0.5)
        outb = torch.empty((N, Cb), device=dev)
        ws = torch.empty(max(1, pr.workspace_bytes(_lib.OP_DIFFUSION_SCALING, 1, N, N, D, 1),
                             pr.workspace_bytes(_lib.OP_GAUSS_SUM_SCALED, 1, N, N, D, Cb)), dtype=torch.uint8, device=dev)
        ts = _events_time(lambda: pr.diffusion_scaling(xs, 0.05, 0.5, workspace=ws), steps, warmup)
        ta = _events_time(lambda: pr.gauss_sum_scaled(xs, xs, vb, 0.05, row_scale=sv, col_scale=sv, out=outb,
                                                      workspace=ws), steps, warmup)
        rows["diffusion_operator_fp32_n131072_d3"] = {"scaling_ms": ts * 1e3, "apply_block4_ms": ta * 1e3,
                                                      "apply_pairs_per_s": float(N) * N / ta}
        if cpu:
            import oracle
            n = 1024
            xh, vh, sh = xs.cpu().numpy(), vb.cpu().numpy(), sv.cpu().numpy()
            rows["diffusion_operator_fp32_n131072_d3"].update(_oracle_rate(
                lambda: oracle.gauss_sum_scaled(xh[:n], xh, vh, 0.05, row_scale=sh[:n], col_scale=sh,
                                                workers=os.cpu_count()),
                float(n) * N, f"one block-4 application, first {n} rows x all {N} columns"))

    # argKmin (K=10) + log-sum-exp, 100k uniform
    if want("argkmin_lse"):
        inp = workloads.make_inputs("argkmin_lse_100k")
        x, y = _resident(inp, ("x", "y"), dev)
        M, N, K = inp["M"], inp["N"], inp["K"]
        sig = float(inp["sigma"])
        idx = torch.empty((M, K), dtype=torch.int32, device=dev)
        lse_out = torch.empty((M,), device=dev)
        ws = torch.empty(max(pr.workspace_bytes(2, 1, M, N, 3, 1, K), pr.workspace_bytes(1, 1, M, N, 3, 1), 1),
                         dtype=torch.uint8, device=dev)

        def argk_lse():
            pr.argkmin(x, y, K, idx=idx, workspace=ws)
            pr.lse(x, y, sig, out=lse_out, workspace=ws)

        t = _events_time(argk_lse, steps, warmup)
        ta = _events_time(lambda: pr.argkmin(x, y, K, idx=idx, workspace=ws), steps, warmup)
        tl = _events_time(lambda: pr.lse(x, y, sig, out=lse_out, workspace=ws), steps, warmup)
        ws2 = torch.empty(max(pr.workspace_bytes(_lib.OP_ARGKMIN_LSE, 1, M, N, 3, 1, K), 1), dtype=torch.uint8,
                          device=dev)
        tf = _events_time(lambda: pr.argkmin_lse(x, y, K, sig, idx=idx, lse_out=lse_out, workspace=ws2), steps, warmup)
        pairs = float(M) * N
        rows["argkmin_lse_100k"] = {"ms": t * 1e3, "argkmin_ms": ta * 1e3, "lse_ms": tl * 1e3,
                                    "fused_ms": tf * 1e3, "pairs_per_s": 2 * pairs / t,
                                    "fused_pairs_per_s": pairs / tf}
        if cpu:
            import oracle
            n = 512

            def oracle_argk_lse():
                oracle.argkmin(inp["x"][:n], inp["y"], K, workers=os.cpu_count())
                oracle.logsumexp_reduction(inp["x"][:n], inp["y"], sig, workers=os.cpu_count())

            rows["argkmin_lse_100k"].update(_oracle_rate(
                oracle_argk_lse, 2.0 * n * N, f"argKmin and LSE, first {n} rows x all {N} columns"))

    # The 1M x 1M Gauss sum with one far row and one far column (near (1000, 1000, 1000)): the
    # two points are set aside and the rest stays on the matrix cores.
    if want("gauss_sum_1m_outliers"):
        inp = workloads.make_inputs("gauss_sum_1m")
        xo, yo = inp["x"].copy(), inp["y"].copy()
        xo[123_457] = 1000.0
        yo[876_543] = np.float32(1000.001)
        x, y, b = (torch.from_numpy(a).to(dev) for a in (xo, yo, inp["b"]))
        M, N = inp["M"], inp["N"]
        out = torch.empty((M, 1), device=dev)
        ws = torch.empty(pr.workspace_bytes(0, 1, M, N, 3, 1), dtype=torch.uint8, device=dev)
        sig = float(inp["sigma"])
        t = _events_time(lambda: pr.gauss_sum(x, y, b, sig, out=out, workspace=ws), max(3, min(steps, 10)), warmup)
        rows["gauss_sum_1m_one_far_row_and_column"] = {"ms": t * 1e3, "pairs_per_s": float(M) * N / t}
        del x, y, b, out, ws

    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-rows", type=int, default=8192, help="rows of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the batched fp16 matrix-core workload reported beside the headline")
    ap.add_argument("--all", action="store_true", help="also time the other workloads")
    ap.add_argument("--only", choices=ALL_GROUPS, default=None,
                    help="with --all: time one group of workloads and skip the headline line")
    ap.add_argument("--all-out", default="bench_all.json")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run one 256 MiB device-to-device copy (the reference kernel that scales the "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this engine has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        a = torch.ones(1 << 26, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": a.numel() * 4}), flush=True)
        return
    if args.all:
        rows = bench_all(args.steps, args.warmup, args.only, cpu=not args.no_cpu_baseline)
        os.makedirs(os.path.dirname(os.path.abspath(args.all_out)), exist_ok=True)
        with open(args.all_out, "w") as f:
            json.dump(rows, f, indent=1)
        for k, v in rows.items():
            print(f"[all] {k}: " + ", ".join(f"{a}={b:.4g}" if isinstance(b, float) else f"{a}={b}"
                                             for a, b in v.items()), file=sys.stderr, flush=True)
        if args.only:
            return
    res = bench_gauss_1m(args.steps, args.warmup, args.cpu_rows, cpu_baseline=not args.no_cpu_baseline)
    if not args.no_secondary:
        res["secondary"] = [bench_fp16_secondary(max(100, args.steps), max(3, args.warmup))]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
