"""torch.autograd glue for the float32 Gauss sum ("Kernel matrix reduction", Variants: each
partial derivative is its own reduction, plugged into torch.autograd).

Forward: keops_gauss_sum. Backward for the upstream gradient g = dL/ds: keops_gauss_sum_grad_x,
keops_gauss_sum_grad_y and keops_gauss_sum_grad_b, each only when its input needs a gradient.
"""
from __future__ import annotations

import torch

from . import gauss_sum, gauss_sum_grad_b, gauss_sum_grad_x, gauss_sum_grad_y


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
        g = g.contiguous()
        gx = gauss_sum_grad_x(x, y, b, g, ctx.sigma) if ctx.needs_input_grad[0] else None
        gy = gauss_sum_grad_y(x, y, b, g, ctx.sigma) if ctx.needs_input_grad[1] else None
        gb = gauss_sum_grad_b(x, y, g, ctx.sigma) if ctx.needs_input_grad[2] else None
        return gx, gy, gb, None
