"""torch.autograd glue for the Gauss sum ("Kernel matrix reduction", Variants: each partial
derivative is its own reduction, plugged into torch.autograd).

Forward: keops_gauss_sum. Backward for the upstream gradient g = dL/ds: one
keops_gauss_sum_backward call computing only the gradients whose inputs need one. Works for
the float32 (M, D) path and the fp16 batched (B, M, D) path; fp16 inputs receive their
gradients cast back to fp16, as autograd requires.
"""
from __future__ import annotations

import torch

from . import gauss_sum, gauss_sum_backward


class GaussSum(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, y, b, sigma):
        x, y, b = x.contiguous(), y.contiguous(), b.contiguous()
        ctx.save_for_backward(x, y, b)
        ctx.sigma = sigma
        return gauss_sum(x, y, b, sigma)

    @staticmethod
    def backward(ctx, g):
        x, y, b = ctx.saved_tensors
        need = tuple(k for k, want in zip(("x", "y", "b"), ctx.needs_input_grad[:3]) if want)
        if not need:
            return None, None, None, None
        grads = gauss_sum_backward(x, y, b, g.to(torch.float32).contiguous(), ctx.sigma, need=need)
        out = []
        for key, t in (("x", x), ("y", y), ("b", b)):
            gk = grads.get(key)
            out.append(None if gk is None else gk.to(t.dtype))
        return out[0], out[1], out[2], None
