"""CPU float64 oracle for the pairwise reductions — test infrastructure, not product code.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this
package. The device library never imports, links or calls it.
"""
from .reductions import (  # noqa: F401
    argkmin,
    argkmin_weighted,
    default_workers,
    diffusion_scaling,
    gauss_sum,
    gauss_sum_batched,
    gauss_sum_batched_backward,
    gauss_sum_grad_b,
    gauss_sum_grad_x,
    gauss_sum_grad_y,
    gauss_sum_scaled,
    keys_are_exact,
    logsumexp_reduction,
    squared_distances,
)
