"""Differentiable solve x = A^-1 b as a torch.autograd.Function.

Forward runs the library's PCG (M^-1 = G G^T + eps I); backward runs the
library's adjoint solve A^T lambda = dL/dx and returns dL/db = lambda and
dL/dvals[k] = -lambda_row(k) x_col(k) on A's stored entries ("torch-sla",
Technical Summary, Methodology 2: one adjoint solve, gradient only on the
sparsity pattern, O(n + nnz) memory independent of the iteration count).
Only x is saved between forward and backward.
"""
from __future__ import annotations

import torch

from . import binding as B


class PCGSolve(torch.autograd.Function):
    @staticmethod
    def forward(ctx, vals, b, A: B.Mat, G: B.Mat, eps: float, rtol: float, maxit: int):
        # `vals` must be the tensor A was created from (the handle borrows it).
        if vals.data_ptr() != A._keep[2].data_ptr():
            raise ValueError("vals must be the value tensor the handle A borrows")
        x, info = B.sla_pcg_solve(A, G, eps, b.contiguous(), rtol=rtol, maxit=maxit)
        ctx.save_for_backward(x)
        ctx.A, ctx.G, ctx.eps, ctx.rtol, ctx.maxit = A, G, eps, rtol, maxit
        ctx.info = info
        return x

    @staticmethod
    def backward(ctx, grad_x):
        (x,) = ctx.saved_tensors
        grad_b, grad_vals, _ = B.sla_pcg_adjoint(ctx.A, ctx.G, ctx.eps, x, grad_x.contiguous(),
                                                 rtol=ctx.rtol, maxit=ctx.maxit)
        return grad_vals, grad_b, None, None, None, None, None


def solve(vals, b, A: B.Mat, G: B.Mat, eps: float = 3e-3, rtol: float = 1e-10,
          maxit: int = 5000):
    """x = A^-1 b, differentiable in A's stored values and in b."""
    return PCGSolve.apply(vals, b, A, G, eps, rtol, maxit)
