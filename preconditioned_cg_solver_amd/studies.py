"""Studies run through the library's kernels (reports, not the hot path).

* ``jacobi``: PCG with the factorised SPAI preconditioner (seeded random G on
  A's lower pattern, eps = 3e-3) against diagonal (Jacobi) preconditioning,
  M^-1 = D^-1 (G = diag(a_ii^-1/2), eps = 0), through the same kernels; and
  an eps sweep (3e-5 ... 3e-1) of the SPAI preconditioner.  This mirrors the
  learned-SPAI page's "Measured effects" table (Diagonal vs SPAI total solve
  time; the eps ablation) on the synthetic workloads -- with a random G,
  not the learned one, so the iteration counts are not the pages'.

* ``quality``: the preconditioner-quality metrics of the learned-SPAI page's
  setup for the same two preconditioners: the condition number of M^-1 A
  estimated from the solve's own CG coefficients (extreme eigenvalues of the
  Lanczos tridiagonal) and the scale-invariant SAI loss
  || A M^-1 / s - I ||_F^2 / n estimated with Rademacher probes, s being the
  mean absolute stored entry of A.

* ``trace``: one forward and one adjoint solve (with dL/dA) of a power-law
  SPD system of ``--rows`` rows (default 20,000) on its locality ordering:
  the run to record with ``SLA_TRACE=1`` under ``rocprofv3 --marker-trace``,
  which shows the library's phases (handle creation, the ordering, the
  solves, the pattern gradient) around their kernels.

Usage: ``python -m preconditioned_cg_solver_amd.studies jacobi|quality|trace
[--configs 0,1,2,3] [--rows N]``.  jacobi and quality print one JSON line per
configuration.
"""
from __future__ import annotations

import argparse
import json
import time

import numpy as np
import torch

from . import binding as B
from . import inputs as I


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _handle(M, transpose=False):
    arrs = (_dev(M.row_ptr), _dev(M.col_idx), _dev(M.vals))
    if M.block_dim == 1:
        return B.sla_csr_create(*arrs, build_transpose=transpose)
    return B.sla_bsr_create(*arrs, block_dim=M.block_dim, build_transpose=transpose)


def _timed_solve(A, G, eps, b, rtol, maxit, work, reps=3):
    x = torch.empty_like(b)
    B.sla_pcg_solve(A, G, eps, b, x=x, rtol=rtol, maxit=maxit, work=work)
    ts, info = [], None
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        _, info = B.sla_pcg_solve(A, G, eps, b, x=x, rtol=rtol, maxit=maxit, work=work)
        ts.append(time.perf_counter() - t0)
    return info, float(np.median(ts))


def jacobi(configs):
    for c in configs:
        p = I.make_problem(c)
        A = _handle(p.A)
        G = _handle(p.G, transpose=True)
        D = _handle(I.diagonal_factor(p.A), transpose=True)
        b = _dev(p.b)
        work = B.workspace(A)
        spai, t_spai = _timed_solve(A, G, p.eps, b, p.rtol, p.maxit, work)
        diag, t_diag = _timed_solve(A, D, 0.0, b, p.rtol, p.maxit, work)
        sweep = {}
        for eps in (3e-5, 3e-4, 3e-3, 3e-2, 3e-1):
            info, t = _timed_solve(A, G, eps, b, p.rtol, p.maxit, work, reps=1)
            sweep[f"{eps:g}"] = {"iterations": info.iterations, "ms": round(t * 1e3, 2),
                                 "status": B.sla_status_string(info.status)}
        print(json.dumps({
            "config": p.name, "n": p.A.n, "nnz": p.A.nnz, "rtol": p.rtol,
            "spai": {"eps": p.eps, "iterations": spai.iterations, "ms": round(t_spai * 1e3, 2)},
            "jacobi": {"iterations": diag.iterations, "ms": round(t_diag * 1e3, 2)},
            "eps_sweep": sweep}), flush=True)
        for h in (A, G, D):
            h.destroy()


def _quality(A, G, eps, b, rtol, maxit, probes, scale):
    _, info, al, be = B.sla_pcg_solve_history(A, G, eps, b, rtol=rtol, maxit=maxit,
                                              raise_on_error=False)
    lo, hi = B.sla_lanczos_extremes(al.numpy(), be.numpy())
    loss = B.sla_sai_loss(A, G, eps, probes, scale)
    n = probes.shape[0]
    return {"iterations": info.iterations, "ritz_min": lo, "ritz_max": hi, "kappa_est": hi / lo,
            "sai_loss_per_n": float(loss.mean().item()) / n}


def quality(configs, nprobe=16):
    for c in configs:
        p = I.make_problem(c)
        A = _handle(p.A)
        G = _handle(p.G, transpose=True)
        D = _handle(I.diagonal_factor(p.A), transpose=True)
        b = _dev(p.b)
        W = np.random.default_rng(1000 + c).choice([-1.0, 1.0], size=(p.A.n, nprobe))
        probes = _dev(W)
        scale = float(np.mean(np.abs(p.A.vals)))
        print(json.dumps({
            "config": p.name, "n": p.A.n, "rtol": p.rtol, "probes": nprobe, "scale": scale,
            "spai": dict(eps=p.eps, **_quality(A, G, p.eps, b, p.rtol, p.maxit, probes, scale)),
            "jacobi": _quality(A, D, 0.0, b, p.rtol, p.maxit, probes, scale)}), flush=True)
        for h in (A, G, D):
            h.destroy()


def trace_run(rows: int):
    """One forward and one adjoint solve of a seeded power-law SPD system
    (16 random neighbours per row, Zipf 2.1 column weights, factorised SPAI
    eps = 3e-3), forced onto its locality ordering."""
    import os
    os.environ.setdefault("SLA_ORDER", "1")
    rng = np.random.default_rng([20, rows])
    A = I.powerlaw_spd(rows, rng)
    G = I.spai_factor(A, rng)
    b = rng.standard_normal(rows)
    dev = torch.device("cuda:0")

    def mk(M, transpose=False):
        return B.sla_csr_create(torch.as_tensor(M.row_ptr.astype(np.int32), device=dev),
                                torch.as_tensor(M.col_idx.astype(np.int32), device=dev),
                                torch.as_tensor(M.vals, device=dev), build_transpose=transpose)
    Ah, Gh = mk(A), mk(G, transpose=True)
    bt = torch.as_tensor(b, device=dev)
    x, info = B.sla_pcg_solve(Ah, Gh, 3e-3, bt, rtol=1e-8, maxit=2000)
    _, _, ainfo = B.sla_pcg_adjoint(Ah, Gh, 3e-3, x, bt, rtol=1e-8, maxit=2000)
    print(json.dumps({"rows": rows, "nnz": int(A.nnz), "reordered": B.sla_mat_reordered(Ah),
                      "iterations": info.iterations, "adjoint_iterations": ainfo.iterations}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("study", choices=["jacobi", "quality", "trace"])
    ap.add_argument("--configs", default="0,1,2,3")
    ap.add_argument("--rows", type=int, default=20000)
    args = ap.parse_args()
    configs = [int(c) for c in args.configs.split(",")]
    if args.study == "jacobi":
        jacobi(configs)
    elif args.study == "quality":
        quality(configs)
    else:
        trace_run(args.rows)


if __name__ == "__main__":
    main()
