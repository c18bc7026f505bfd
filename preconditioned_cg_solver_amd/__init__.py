"""MI355X (gfx950) preconditioned conjugate gradients with a factorised sparse
approximate inverse M^-1 = G G^T + eps I, forward and adjoint.

The numerical work lives in ``libsla.so`` (hand-written HIP kernels behind the
C ABI of ``include/sla.h``); ``binding`` marshals torch tensors to it and
``autograd`` wraps forward + adjoint as a torch.autograd.Function.  ``inputs``
holds the seeded synthetic workloads.  Submodules that need the library load
it on first use and raise if it has not been built.
"""

__all__ = ["binding", "autograd", "inputs", "build"]
