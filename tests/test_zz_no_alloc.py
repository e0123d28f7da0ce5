"""The allocation-free Gauss sum (keops_gauss_sum_noalloc) against the workspace entry point
keops_gauss_sum, through the C ABI: two calls in a row on the same device, the second on a
smaller input (the scratch array keeps the first call's contents), must give bit-identical
outputs, and both must meet the oracle's float32 bar on sampled rows."""
import ctypes

import numpy as np
import pytest

import oracle
from pairwise_reductions_amd import _lib, workloads

pytestmark = pytest.mark.gpu


def _case(seed, M, N, D, C):
    rng = np.random.default_rng(seed)
    x = workloads.grid24(rng, (M, D))
    y = workloads.grid24(rng, (N, D))
    b = rng.standard_normal((N, C)).astype(np.float32)
    return x, y, b


def test_noalloc_matches_workspace_entry_point_twice():
    import torch
    import pairwise_reductions_amd as pr
    lib = _lib.load()
    stream = torch.cuda.current_stream().cuda_stream
    # the second call is smaller than the first
    for seed, (M, N, D, C, sigma) in enumerate([(120_000, 150_000, 3, 1, 0.02), (3_001, 5_003, 3, 2, 0.1)]):
        print(f"[case] noalloc seed={seed} M={M} N={N} D={D} C={C}", flush=True)
        x, y, b = _case(seed, M, N, D, C)
        xd, yd, bd = (torch.from_numpy(a).cuda() for a in (x, y, b))
        sig = float(np.float32(sigma))
        ref = pr.gauss_sum(xd, yd, bd, sig)
        out = torch.full((M, C), float("nan"), dtype=torch.float32, device="cuda")
        st = lib.keops_gauss_sum_noalloc(xd.data_ptr(), yd.data_ptr(), bd.data_ptr(), out.data_ptr(), 1, M, N, D, C,
                                         ctypes.c_float(sig), _lib.KEOPS_F32, stream)
        assert st == 0, lib.keops_last_error()
        torch.cuda.synchronize()
        got, want_dev = out.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(got, want_dev), "allocation-free and workspace entry points differ"
        rows = workloads.sample_rows(M, 256, seed=seed)
        want, norm = oracle.gauss_sum(x[rows], y, b, sig, workers=8)
        err = float(np.max(np.abs(got[rows].astype(np.float64) - want) / norm))
        assert err <= 1e-4, f"normalised error {err:.3e}"


def test_noalloc_fp16_and_odd_width():
    """The matrix-core family through the same scratch (fp16, D = 20 padded inside it)."""
    import torch
    import pairwise_reductions_amd as pr
    print("[case] noalloc fp16 B=2 M=700 N=1500 D=20 C=4", flush=True)
    g = torch.Generator().manual_seed(7)
    q = (torch.randn((2, 700, 20), generator=g) / 20 ** 0.5).half().cuda()
    k = (torch.randn((2, 1500, 20), generator=g) / 20 ** 0.5).half().cuda()
    v = torch.randn((2, 1500, 4), generator=g).half().cuda()
    ref = pr.gauss_sum(q, k, v, 1.0)
    out = torch.empty_like(ref)
    pr.gauss_sum_noalloc(q, k, v, 1.0, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_noalloc_refuses_sizes_beyond_the_scratch():
    import torch
    import pairwise_reductions_amd as pr
    x = torch.zeros((600_000, 3), device="cuda")
    b = torch.zeros((600_000, 1), device="cuda")
    out = torch.empty((600_000, 1), device="cuda")
    with pytest.raises(pr.KeopsError, match="scratch"):
        pr.gauss_sum_noalloc(x, x, b, 0.01, out)
