"""Compile the HIP sources into the in-tree shared library libkeops_mi355x.so (gfx950).

Each source is compiled on its own (in parallel) and then linked with hipcc. The library
is always rebuilt when build() is called.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libkeops_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
HIGHD_SOURCES = ["highd.hip", "highd_d32.hip", "highd_d64.hip", "highd_d96.hip", "highd_d128.hip"]
SOURCES = ["abi.hip", "lowd.hip", "lowd_sum.hip", "lowd_mfma.hip", "lowd_lse.hip", "lowd_knn.hip", "lowd_grad.hip"] + HIGHD_SOURCES
# Per-source extras. The matrix-core sources keep matrix-core accumulators in ordinary VGPRs (the
# exponent and max steps read every accumulator value, so AGPR copies would cost a VALU op
# each) and runs with IEEE mode off, so max needs no NaN quieting.
EXTRA_FLAGS = {src: ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mno-amdgpu-ieee", "-fno-honor-nans"]
               for src in HIGHD_SOURCES}
EXTRA_FLAGS["lowd_mfma.hip"] = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA_FLAGS["lowd_knn.hip"] = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
ARCH = os.environ.get("KEOPS_OFFLOAD_ARCH", "gfx950")

# Packed-FP32 instruction selection is switched off: every float32 op is a plain VALU op.
COMMON_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-I" + INCLUDE, "-I" + CSRC,
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in proc.stdout.splitlines()
                    if "is not a recognized feature for this target" not in line)
    if proc.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (proc.returncode, " ".join(cmd), out))
    return out


def build(verbose: bool = False) -> str:
    """Build the library in-tree and return its path."""
    hipcc = _hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        jobs.append((obj, [hipcc, *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]))
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    tmp = LIB_PATH + ".tmp"
    outs.append(_run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + [j[0] for j in jobs]))
    os.replace(tmp, LIB_PATH)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
