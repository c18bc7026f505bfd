"""GPU parity of the several-right-hand-side path (k solves sharing A and G)
against the CPU oracle's column-by-column solves.

Gates: products Y = A X within 1e-13 relative per column (fp64); every
column's solution within 1e-8 of the oracle's solve of that column and its
iteration count within 2 % (at least 1) -- or, where the oracle's own
stopping iteration moves by more under one-ulp perturbations of that column,
within that spread (+-1) and 10x its solution spread; per-column statuses
equal; adjoint
dL/dB and the pattern gradient summed over the solves within 1e-7; the
summed gradient bit-exact against the same sum taken on the host from the
device's Lambda and X.
"""
import numpy as np
import pytest
import torch

import oracle
from preconditioned_cg_solver_amd import binding as B
from preconditioned_cg_solver_amd import inputs as I
from gpu_util import (DEV, assert_solve_matches, create, host, iters_close, problem, rel, say,
                      tdev)

pytestmark = pytest.mark.gpu

ORC_TO_SLA = {oracle.OK: B.OK, oracle.NOT_CONVERGED: B.NOT_CONVERGED,
              oracle.ERR_BREAKDOWN: B.ERR_BREAKDOWN, oracle.ERR_NONFINITE: B.ERR_NONFINITE}


@pytest.fixture(params=["sliced", "rows"])
def layout(request, monkeypatch):
    """The sliced layouts (SELL-64, BSR sliced ELL) or the plain row engine."""
    if request.param == "rows":
        monkeypatch.setenv("SLA_SELL", "0")
    return request.param


@pytest.fixture(params=["separate", "fused"])
def form(request, monkeypatch):
    """The iteration's two forms: single-gather products with separate vector
    passes, or p and r formed inside the products' gathers.  (With the
    default form, systems of at most 1024 rows take one workgroup per column;
    the fused form keeps them in lock step.)"""
    if request.param == "fused":
        monkeypatch.setenv("SLA_MFUSION", "fused")
        monkeypatch.setenv("SLA_SMALL", "0")
    return request.param


def rhs(n, k, seed):
    return np.random.default_rng(seed).standard_normal((n, k))


MATS = ["c0", "poisson3d_13", "bsr_elastic_6", "powerlaw_20k", "irregular_long_rows"]


@pytest.mark.parametrize("key", MATS)
@pytest.mark.parametrize("k", [1, 2, 3, 8, 11])
def test_spmm_parity(key, k, layout):
    p = problem(key)
    X = rhs(p.A.n, k, 5)
    say("spmm", key, k, layout)
    A = create(p.A, transpose=True)
    Y = host(B.sla_spmm(A, tdev(X)))
    Yt = host(B.sla_spmm_t(A, tdev(X)))
    trp, tci, tv = oracle.transpose(p.A)
    At = I.SparseMatrix(p.A.n_block_rows, p.A.block_dim, trp, tci, tv)
    for c in range(k):
        ref = oracle.spmv(p.A, X[:, c])
        assert rel(Y[:, c], ref) <= 1e-13, ("column", c)
        assert rel(Yt[:, c], oracle.spmv(At, X[:, c])) <= 1e-13, ("transposed column", c)


def test_spmm_empty_and_errors():
    p = problem("c0")
    A = create(p.A)
    say("spmm k = 0 and bad arguments")
    e = torch.empty(p.A.n, 0, dtype=torch.float64, device=DEV)
    B.sla_spmm(A, e, torch.empty_like(e))
    X = tdev(rhs(p.A.n, 2, 1))
    with pytest.raises(B.SlaError):
        B.sla_spmm(A, X, X)
    with pytest.raises(B.SlaError):
        B.sla_spmm_t(A, X)  # no transpose built


_oracle_cache = {}


def check_solve(p, Bm, rtol, maxit, cache_key=None):
    if cache_key is not None and cache_key in _oracle_cache:
        Xr, st_r, it_r, rr_r, sts_r = _oracle_cache[cache_key]
    else:
        Xr, st_r, it_r, rr_r, sts_r = oracle.pcg_multi(p.A, p.G, p.eps, Bm, rtol, maxit)
        if cache_key is not None:
            _oracle_cache[cache_key] = (Xr, st_r, it_r, rr_r, sts_r)
    A, G = create(p.A), create(p.G, transpose=True)
    X, infos = B.sla_pcg_solve_multi(A, G, p.eps, tdev(Bm), rtol=rtol, maxit=maxit,
                                     raise_on_error=False)
    Xg = host(X)
    for c in range(Bm.shape[1]):
        assert infos[c].status == ORC_TO_SLA[int(sts_r[c])], (c, infos[c], sts_r[c])
        # outside the fixed gates only within the oracle's own rounding spread
        assert_solve_matches(p.A, p.G, p.eps, Bm[:, c], rtol, maxit, infos[c].iterations,
                             Xg[:, c], int(it_r[c]), Xr[:, c], strict=False,
                             what="column %d" % c)
    return Xg, infos


@pytest.mark.parametrize("key", MATS)
@pytest.mark.parametrize("k", [2, 5, 8])
def test_solve_multi_parity(key, k, layout, form):
    p = problem(key)
    Bm = rhs(p.A.n, k, 7)
    Bm[:, 0] = p.b
    if k > 2:
        Bm[:, 2] = 0.0            # solved at once with x = 0
        Bm[:, 1] *= 1e-3          # same iterations as an unscaled column
    say("solve_multi", key, k, layout, form, p.A.n)
    check_solve(p, Bm, p.rtol, p.maxit, cache_key=(key, k))


def test_solve_multi_columns_exit_at_different_iterations():
    """With a scalar preconditioner an eigenvector column converges in one
    iteration while the others continue; its x must stay as it was."""
    N = 16
    A = I.poisson2d(N)
    Gs = I.SparseMatrix(A.n, 1, np.arange(A.n + 1, dtype=np.int32),
                        np.arange(A.n, dtype=np.int32), np.full(A.n, 0.7))
    i, j = np.meshgrid(np.arange(1, N + 1), np.arange(1, N + 1), indexing="ij")
    v = (np.sin(3 * np.pi * i / (N + 1)) * np.sin(5 * np.pi * j / (N + 1))).reshape(-1)
    Bm = np.stack([v, np.random.default_rng(3).standard_normal(A.n), 2 * v,
                   np.random.default_rng(4).standard_normal(A.n)], axis=1)
    p = I.Problem("eig", -1, A, Gs, Bm[:, 0], 3e-3, 1e-12, 500, "dot", None)
    say("solve_multi eigenvector columns")
    _, infos = check_solve(p, Bm, 1e-12, 500)
    assert infos[0].iterations == 1 and infos[2].iterations == 1
    assert infos[1].iterations > 20 and infos[3].iterations > 20


def test_solve_multi_edges(form):
    p = problem("c0")
    n = p.A.n
    Bm = rhs(n, 4, 9)
    Bm[5, 1] = np.nan
    say("solve_multi NaN column, maxit 0 and 3")
    A, G = create(p.A), create(p.G, transpose=True)
    X, infos = B.sla_pcg_solve_multi(A, G, p.eps, tdev(Bm), rtol=p.rtol, maxit=p.maxit,
                                     raise_on_error=False)
    assert infos[1].status == B.ERR_NONFINITE and infos[1].iterations == 0
    assert not torch.any(X[:, 1])
    Xr, _, it_r, _, _ = oracle.pcg_multi(p.A, p.G, p.eps, Bm[:, [0, 2, 3]], p.rtol, p.maxit)
    for c, cr in ((0, 0), (2, 1), (3, 2)):
        assert infos[c].status == B.OK and iters_close(infos[c].iterations, int(it_r[cr]))
        assert rel(host(X[:, c]), Xr[:, cr]) <= 1e-8
    with pytest.raises(B.SlaError):
        B.sla_pcg_solve_multi(A, G, p.eps, tdev(Bm), rtol=p.rtol, maxit=p.maxit)
    Bm[5, 1] = 1.0
    X, infos = B.sla_pcg_solve_multi(A, G, p.eps, tdev(Bm), rtol=p.rtol, maxit=0,
                                     raise_on_error=False)
    assert all(i.status == B.NOT_CONVERGED and i.iterations == 0 for i in infos)
    assert not torch.any(X)
    check_solve(p, Bm, p.rtol, 3)


def test_solve_multi_fp32_heat():
    """fp32 storage and products, fp64 scalars: closeness to the fp64 solves."""
    p = problem("heat2d_64")
    Bm = rhs(p.A.n, 4, 11)
    Xr, _, _, _, _ = oracle.pcg_multi(p.A, p.G, p.eps, Bm, p.rtol, p.maxit)
    p32 = p.astype("f32")
    say("solve_multi fp32 heat", p.A.n)
    A, G = create(p32.A, dtype="f32"), create(p32.G, transpose=True, dtype="f32")
    X, infos = B.sla_pcg_solve_multi(A, G, p.eps, tdev(Bm, torch.float32), rtol=p.rtol,
                                     maxit=p.maxit, raise_on_error=False)
    assert all(i.status in (B.OK, B.NOT_CONVERGED) for i in infos)
    assert rel(host(X), Xr) <= 1e-3


@pytest.mark.parametrize("key", ["c0", "bsr_elastic_6", "powerlaw_20k"])
def test_adjoint_multi_parity(key, layout, form):
    p = problem(key)
    k = 3
    Bm = rhs(p.A.n, k, 13)
    W = rhs(p.A.n, k, 14)
    Xr, _, _, _, _ = oracle.pcg_multi(p.A, p.G, p.eps, Bm, p.rtol, p.maxit)
    lam_r, g_r, st_r, it_r, _, _ = oracle.adjoint_multi(p.A, p.G, p.eps, Xr, W, p.rtol, p.maxit)
    assert st_r == oracle.OK
    say("adjoint_multi", key, layout, p.A.n)
    A, G = create(p.A), create(p.G, transpose=True)
    X, _ = B.sla_pcg_solve_multi(A, G, p.eps, tdev(Bm), rtol=p.rtol, maxit=p.maxit)
    GB, gv, infos = B.sla_pcg_adjoint_multi(A, G, p.eps, X, tdev(W), rtol=p.rtol, maxit=p.maxit)
    for c in range(k):
        assert infos[c].status == B.OK and iters_close(infos[c].iterations, int(it_r[c]))
    lam, x = host(GB), host(X)
    assert rel(lam, lam_r) <= 1e-7
    assert rel(host(gv), g_r) <= 1e-7
    # the summed gradient from the device's own Lambda and X, same order
    rows = p.A.row_of_entry()
    bs = p.A.block_dim
    if bs == 1:
        ri, cj = rows, p.A.col_idx
    else:
        e = np.arange(p.A.nnz)
        kb, w = e // 9, e % 9
        ri, cj = 3 * rows[kb] + w // 3, 3 * p.A.col_idx[kb] + w % 3
    g = np.zeros(p.A.nnz)
    for c in range(k):
        g = g - lam[ri, c] * x[cj, c]
    assert np.array_equal(host(gv), g)


@pytest.mark.parametrize("k", [4, 8])
@pytest.mark.parametrize("key", ["c2", "c1", "c3"])
def test_solve_multi_full_size(key, k):
    """The benchmark's several-right-hand-side lines at their size: 3D Poisson
    128^3 (n = 2,097,152), heat 512^2 (n = 262,144) and the elasticity BSR3
    system (n = 786,432), columns N(0, 1) from seed 100 + k with the single
    solve's b as column 0, every column against the oracle's solve of it
    under the fixed gates (x within 1e-8, iterations within 2%)."""
    p = problem(key)
    Bm = np.random.default_rng(100 + k).standard_normal((p.A.n, k))
    Bm[:, 0] = p.b
    say("solve_multi full size", key, p.A.n, k)
    A, G = create(p.A, validate=False), create(p.G, transpose=True, validate=False)
    X, infos = B.sla_pcg_solve_multi(A, G, p.eps, tdev(Bm), rtol=p.rtol, maxit=p.maxit)
    Xg = host(X)
    Xr, st_r, it_r, _, sts_r = oracle.pcg_multi(p.A, p.G, p.eps, Bm, p.rtol, p.maxit)
    assert st_r == oracle.OK
    for c in range(k):
        say("  column", c, "iterations gpu", infos[c].iterations, "oracle", int(it_r[c]))
        assert infos[c].status == B.OK and infos[c].converged
        assert iters_close(infos[c].iterations, int(it_r[c])), (c, infos[c].iterations, it_r[c])
        assert rel(Xg[:, c], Xr[:, c]) <= 1e-8, (c, rel(Xg[:, c], Xr[:, c]))


@pytest.mark.parametrize("k", [5, 11])
def test_solve_multi_passes_on_a_far_reaching_matrix(k):
    """3D Poisson 92^3 reaches 8,464 rows from its diagonal, so its columns
    run in passes of at most 4 with each pass's X kept in the workspace
    (k = 5: 4 + 1, k = 11: 4 + 4 + 2 + 1); every column against the oracle's
    solve of it, and the adjoint's dL/dB and summed dL/dA."""
    p = problem("poisson3d_92")
    Bm = rhs(p.A.n, k, 31)
    say("solve_multi passes, far-reaching matrix", k, p.A.n)
    Xg, infos = check_solve(p, Bm, p.rtol, p.maxit)
    W = rhs(p.A.n, k, 32)
    A, G = create(p.A, validate=False), create(p.G, transpose=True, validate=False)
    GB, gv, ainfos = B.sla_pcg_adjoint_multi(A, G, p.eps, tdev(Xg), tdev(W), rtol=p.rtol,
                                             maxit=p.maxit)
    Xr, _, _, _, _ = oracle.pcg_multi(p.A, p.G, p.eps, Bm, p.rtol, p.maxit)
    lam, gval, st, _, _, _ = oracle.adjoint_multi(p.A, p.G, p.eps, Xr, W, p.rtol, p.maxit)
    assert st == oracle.OK
    assert rel(host(GB), lam) <= 1e-7
    assert rel(host(gv), gval) <= 1e-7
