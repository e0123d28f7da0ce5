"""Benchmark: Gaussian kernel sum pair evaluations per second on one MI355X.

One step is one call of keops_gauss_sum on inputs already resident in HBM: the column-prep
kernel plus the fused reduction kernel over all M x N pairs. The default workload is the
1M x 1M, D=3, C=1, float32, sigma=0.01 Gauss sum. Timing uses HIP events recorded on the
stream the kernels run on, after W warm-up steps, bracketed by device synchronisations.

Prints ONE JSON line (the contract), with two extra objects:
  roofline      the dominant kernel against the float32 vector peak (ALU-bound)
  cpu_baseline  the float64 CPU oracle on a bounded row sample of the same workload
--all additionally times the other workloads and writes them to --all-out (not the line).
"""
from __future__ import annotations

import argparse
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


def _events_time(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps  # seconds per step


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

    t = _events_time(step, steps, warmup)
    pairs = float(M) * float(N)
    flops = pairs * gauss_flops_per_pair(D, C)
    achieved = flops / t / 1e12
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
        "dtype": "f32 (exponent in f64)",
        "data": "synthetic: x, y uniform on the 2^-24 grid in [0,1)^3, b ~ N(0,1), seed 0",
        "config": {"workload": key, "M": M, "N": N, "D": D, "C": C, "sigma": sigma,
                   "pairs_per_step": pairs},
        "roofline": {
            "bound": "alu",
            "achieved": achieved,
            "peak": PEAK_FP32_VECTOR_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_VECTOR_TFLOPS,
            "traffic": None,
            "kernel": "gauss_sum_kernel<3,1,4>",
            "flop_per_pair": gauss_flops_per_pair(D, C),
            "kernel_ms": t * 1e3,
        },
    }
    if cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_gauss(inp, cpu_rows)
    out_host = out.cpu().numpy()
    result["config"]["checksum"] = float(np.sum(out_host, dtype=np.float64))
    return result


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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-rows", type=int, default=2048, help="rows of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this engine has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    res = bench_gauss_1m(args.steps, args.warmup, args.cpu_rows, cpu_baseline=not args.no_cpu_baseline)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
