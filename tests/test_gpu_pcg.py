"""GPU parity of the PCG forward solve and the adjoint solve against the CPU
oracle, plus the stopping-rule edge cases, failure statuses, determinism and
the memory property of the adjoint.

Gates: solution ||x_gpu - x_ref|| / ||x_ref|| <= 1e-8, iteration count within
2 % (at least 1), adjoint gradients dL/db and dL/dA within 1e-7 relative.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from preconditioned_cg_solver_amd import autograd as AG
from preconditioned_cg_solver_amd import binding as B
from preconditioned_cg_solver_amd import inputs as I
from gpu_util import (DEV, assert_iterations_match, assert_solve_matches, create, host,
                      iters_close, oracle_self_sensitivity, problem, rel, say, tdev)

pytestmark = pytest.mark.gpu

def handles(p, dtype="f64"):
    return create(p.A, dtype=dtype), create(p.G, transpose=True, dtype=dtype)


FORWARD = ["c0", "poisson2d_37", "poisson3d_13", "irregular_long_rows", "bsr_elastic_6",
           "powerlaw_20k", "c1", "c2"]
# the benchmark workloads keep the fixed gates (iterations within 2%, x within
# 1e-8) without exception; the other matrices may fall back to the oracle's own
# rounding spread (assert_solve_matches)
STRICT = ("c0", "c1", "c2")


@pytest.fixture(params=["auto", "fused", "unfused"])
def fusion(request, monkeypatch):
    """The iteration's two forms: p and r formed inside the products'
    gathers, or separate vector passes (the library picks per matrix, and
    solves systems of at most 1024 rows in one workgroup)."""
    if request.param != "auto":
        # the explicit forms also keep small systems off the one-workgroup solver
        monkeypatch.setenv("SLA_FUSION", request.param)
        monkeypatch.setenv("SLA_SMALL", "0")
    return request.param


@pytest.mark.parametrize("key", FORWARD)
def test_forward_parity(key, fusion):
    if fusion != "auto" and key in ("c1", "c2"):
        pytest.skip("full-size configs run in the library's own choice only")
    p = problem(key)
    x_ref, st_ref, it_ref, rr_ref = oracle.pcg(p.A, p.G, p.eps, p.b, p.rtol, p.maxit)
    assert st_ref == oracle.OK
    say("pcg forward", key, "n", p.A.n, "oracle iterations", it_ref)
    A, G = handles(p)
    x, info = B.sla_pcg_solve(A, G, p.eps, tdev(p.b), rtol=p.rtol, maxit=p.maxit)
    say("  gpu iterations", info.iterations, "relres", info.rel_residual)
    assert info.status == B.OK and info.converged
    assert info.rel_residual <= p.rtol
    assert_solve_matches(p.A, p.G, p.eps, p.b, p.rtol, p.maxit, info.iterations, host(x),
                         it_ref, x_ref, strict=key in STRICT, what="forward " + key)


@pytest.mark.parametrize("key", ["c0", "poisson3d_13", "bsr_elastic_6", "irregular_long_rows",
                                 "powerlaw_20k", "c2"])
def test_adjoint_parity(key, fusion):
    if fusion != "auto" and key == "c2":
        pytest.skip("full-size configs run in the library's own choice only")
    p = problem(key)
    x_ref, st, it, _ = oracle.pcg(p.A, p.G, p.eps, p.b, p.rtol, p.maxit)
    gx_ref = I.loss_grad_weights(p, x_ref)
    lam_ref, gv_ref, st2, it2, _ = oracle.adjoint(p.A, p.G, p.eps, x_ref, gx_ref, p.rtol, p.maxit)
    assert st == st2 == oracle.OK
    say("pcg adjoint", key, "oracle iterations", it2)
    A, G = handles(p)
    x, info = B.sla_pcg_solve(A, G, p.eps, tdev(p.b), rtol=p.rtol, maxit=p.maxit)
    gx = 2.0 * x if p.loss == "sumsq" else tdev(p.w)
    grad_b, grad_vals, ainfo = B.sla_pcg_adjoint(A, G, p.eps, x, gx, rtol=p.rtol, maxit=p.maxit)
    say("  gpu adjoint iterations", ainfo.iterations)
    assert ainfo.status == B.OK
    assert_iterations_match(p.A, p.G, p.eps, gx_ref, p.rtol, p.maxit, ainfo.iterations, it2,
                            strict=key in STRICT, what="adjoint " + key)
    assert rel(host(grad_b), lam_ref) <= 1e-7
    assert rel(host(grad_vals), gv_ref) <= 1e-7


def test_fp32_heat_runs():
    """fp32 storage and products, fp64 scalars: reported, gated on the
    recursive residual and on closeness to the fp64 solution."""
    p = problem("c1")
    p32 = p.astype("f32")
    x64, st, it64, _ = oracle.pcg(p.A, p.G, p.eps, p.b, p.rtol, p.maxit)
    say("pcg fp32 heat, oracle fp64 iterations", it64)
    A, G = handles(p32, dtype="f32")
    x, info = B.sla_pcg_solve(A, G, p.eps, tdev(p32.b), rtol=p.rtol, maxit=p.maxit)
    say("  gpu fp32 iterations", info.iterations, "status", info.status, "relres",
        info.rel_residual)
    assert info.status in (B.OK, B.NOT_CONVERGED)
    assert rel(host(x), x64) <= 1e-3


def test_edge_zero_rhs():
    p = problem("c0")
    A, G = handles(p)
    say("b = 0")
    x, info = B.sla_pcg_solve(A, G, p.eps, torch.zeros(p.A.n, dtype=torch.float64, device=DEV),
                              rtol=1e-10, maxit=100)
    assert info.status == B.OK and info.iterations == 0 and info.converged
    assert not torch.any(x)


@pytest.mark.parametrize("key", ["c0", "powerlaw_20k"])
def test_edge_maxit_zero_and_small(key, fusion):
    p = problem(key)
    A, G = handles(p)
    b = tdev(p.b)
    say("maxit = 0")
    x, info = B.sla_pcg_solve(A, G, p.eps, b, rtol=1e-10, maxit=0)
    assert info.status == B.NOT_CONVERGED and info.iterations == 0 and not torch.any(x)
    for m in (1, 2, 5, 17):
        say("maxit =", m)
        x, info = B.sla_pcg_solve(A, G, p.eps, b, rtol=1e-10, maxit=m)
        x_ref, st, it, rr = oracle.pcg(p.A, p.G, p.eps, p.b, 1e-10, m)
        assert st == oracle.NOT_CONVERGED and info.status == B.NOT_CONVERGED
        assert info.iterations == it == m
        # iterates agree to rounding; on an ill-conditioned system CG amplifies
        # rounding, so the bound is 100x the oracle's own movement under a
        # one-ulp perturbation of b (about 1e-16 for Poisson, 1.7e-5 at
        # iteration 17 for the power-law system, kappa ~ 1e8)
        sx, sr = oracle_self_sensitivity(p.A, p.G, p.eps, p.b, 1e-10, m)
        assert rel(host(x), x_ref) <= max(1e-12, 100 * sx)
        assert abs(info.rel_residual - rr) <= max(1e-10, 100 * sr) * rr


def test_edge_breakdown_negative_definite(fusion):
    p = problem("c0")
    neg = I.SparseMatrix(p.A.n_block_rows, 1, p.A.row_ptr, p.A.col_idx, -p.A.vals)
    x_ref, st, it, _ = oracle.pcg(neg, p.G, p.eps, p.b, 1e-10, 100)
    assert st == oracle.ERR_BREAKDOWN
    A = create(neg)
    G = create(p.G, transpose=True)
    say("breakdown")
    x, info = B.sla_pcg_solve(A, G, p.eps, tdev(p.b), rtol=1e-10, maxit=100,
                              raise_on_error=False)
    assert info.status == B.ERR_BREAKDOWN and info.iterations == it == 0
    assert rel(host(x), x_ref) == 0.0


def test_edge_nonfinite_rhs():
    p = problem("c0")
    A, G = handles(p)
    b = p.b.copy()
    b[17] = np.nan
    say("NaN in b")
    x, info = B.sla_pcg_solve(A, G, p.eps, tdev(b), rtol=1e-10, maxit=100, raise_on_error=False)
    assert info.status == B.ERR_NONFINITE


def test_edge_one_unknown():
    A = I.SparseMatrix(1, 1, np.array([0, 1], np.int32), np.array([0], np.int32), np.array([4.0]))
    G = I.SparseMatrix(1, 1, np.array([0, 1], np.int32), np.array([0], np.int32), np.array([0.5]))
    say("n = 1")
    x, info = B.sla_pcg_solve(create(A), create(G, transpose=True), 3e-3,
                              tdev(np.array([2.0])), rtol=1e-12, maxit=10)
    assert info.status == B.OK and info.iterations == 1
    assert abs(host(x)[0] - 0.5) <= 1e-16


def test_invalid_arguments():
    p = problem("c0")
    A, G = handles(p)
    b = tdev(p.b)
    say("invalid arguments")
    G_no_t = create(p.G)
    with pytest.raises(B.SlaError) as e:
        B.sla_pcg_solve(A, G_no_t, p.eps, b)
    assert e.value.status == B.ERR_INVALID_ARG
    with pytest.raises(B.SlaError) as e:
        B.sla_pcg_solve(A, G, -1.0, b)
    assert e.value.status == B.ERR_INVALID_ARG
    with pytest.raises(B.SlaError) as e:
        B.sla_pcg_solve(A, G, p.eps, b, x=b)
    assert e.value.status == B.ERR_INVALID_ARG
    small = torch.empty(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(B.SlaError) as e:
        B.sla_pcg_solve(A, G, p.eps, b, work=small)
    assert e.value.status == B.ERR_INVALID_ARG
    other = create(problem("poisson2d_37").G, transpose=True)
    with pytest.raises(ValueError):
        B.sla_pcg_solve(A, other, p.eps, b)      # the binding's check
    # the library's own check, through the raw C ABI
    x = torch.empty_like(b)
    work = B.workspace(A)
    si = B.SolveInfo()
    st = B.lib().sla_pcg_solve(A.handle, other.handle, p.eps, B._ptr(b), B._ptr(x), 1e-10, 10,
                               B._ptr(work), work.numel(), None, ctypes.byref(si))
    assert st == B.ERR_INVALID_ARG
    # lambda (grad_b) may not share memory with x in the adjoint
    x, _ = B.sla_pcg_solve(A, G, p.eps, b, rtol=p.rtol, maxit=p.maxit)
    gv = torch.empty(p.A.nnz, dtype=torch.float64, device=DEV)
    st = B.lib().sla_pcg_adjoint(A.handle, G.handle, p.eps, B._ptr(x), B._ptr(b), B._ptr(x),
                                 B._ptr(gv), 1e-10, 10, B._ptr(work), work.numel(), None,
                                 ctypes.byref(si))
    assert st == B.ERR_INVALID_ARG


@pytest.mark.parametrize("key", ["c0", "irregular_long_rows", "bsr_elastic_6", "powerlaw_20k"])
def test_bitwise_deterministic(key, fusion):
    p = problem(key)
    A, G = handles(p)
    b = tdev(p.b)
    say("determinism", key)
    x1, i1 = B.sla_pcg_solve(A, G, p.eps, b, rtol=p.rtol, maxit=p.maxit)
    x2, i2 = B.sla_pcg_solve(A, G, p.eps, b, rtol=p.rtol, maxit=p.maxit)
    assert i1.iterations == i2.iterations
    assert torch.equal(x1, x2)


def test_adjoint_memory_independent_of_iterations():
    """The adjoint keeps O(n + nnz) state: the same workspace serves any maxit
    and no device memory is taken during the solves."""
    p = problem("poisson3d_13")
    A, G = handles(p)
    b = tdev(p.b)
    work = B.workspace(A)
    size = B.sla_pcg_workspace_size(A)
    x, _ = B.sla_pcg_solve(A, G, p.eps, b, rtol=1e-12, maxit=5000, work=work)
    gx = tdev(p.w)
    B.sla_pcg_adjoint(A, G, p.eps, x, gx, rtol=1e-12, maxit=5000, work=work)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for m in (3, 50, 5000):
        say("adjoint memory, maxit", m)
        B.sla_pcg_adjoint(A, G, p.eps, x, gx, rtol=1e-12, maxit=m, work=work,
                          grad_b=torch.empty_like(x),
                          grad_vals=torch.empty(A.nnz, dtype=torch.float64, device=DEV))
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0
    assert B.sla_pcg_workspace_size(A) == size


def test_autograd_function_matches_oracle():
    p = problem("poisson2d_37")
    vals = tdev(p.A.vals).requires_grad_(False)
    A = B.sla_csr_create(tdev(p.A.row_ptr), tdev(p.A.col_idx), vals, validate=True)
    G = create(p.G, transpose=True)
    v = vals.clone().requires_grad_(True)
    # the handle borrows `vals`; pass the same storage through autograd
    v.data = vals
    b = tdev(p.b).requires_grad_(True)
    say("autograd")
    x = AG.solve(v, b, A, G, eps=p.eps, rtol=1e-12, maxit=5000)
    loss = (x * x).sum()
    loss.backward()
    x_ref, st, it, _ = oracle.pcg(p.A, p.G, p.eps, p.b, 1e-12, 5000)
    lam, gv, st2, _, _ = oracle.adjoint(p.A, p.G, p.eps, x_ref, 2 * x_ref, 1e-12, 5000)
    assert rel(host(x), x_ref) <= 1e-8
    assert rel(host(b.grad), lam) <= 1e-7
    assert rel(host(v.grad), gv) <= 1e-7


@pytest.mark.parametrize("key", ["c0", "poisson3d_13", "bsr_elastic_6", "powerlaw_20k"])
def test_jacobi_parity(key):
    """Diagonal (Jacobi) preconditioning through the same kernels:
    G = diag(a_ii^-1/2), eps = 0, so M^-1 = D^-1."""
    p = problem(key)
    D = I.diagonal_factor(p.A)
    x_ref, st, it, _ = oracle.pcg(p.A, D, 0.0, p.b, p.rtol, p.maxit)
    assert st == oracle.OK
    say("jacobi", key, "oracle iterations", it)
    A = create(p.A)
    Dh = create(D, transpose=True)
    x, info = B.sla_pcg_solve(A, Dh, 0.0, tdev(p.b), rtol=p.rtol, maxit=p.maxit)
    assert info.status == B.OK and iters_close(info.iterations, it)
    assert rel(host(x), x_ref) <= 1e-8


SMALL = {
    "poisson2d_20": lambda: I.make_problem(0, size=20),
    "poisson2d_32": lambda: I.make_problem(0),
    "heat2d_31": lambda: I.make_problem(1, size=31),
    "poisson3d_10": lambda: I.make_problem(2, size=10),
}


@pytest.mark.parametrize("key", list(SMALL))
@pytest.mark.parametrize("small", ["one_workgroup", "multi_kernel"])
def test_small_systems(key, small, monkeypatch):
    """Systems of at most 1024 rows run in one workgroup unless SLA_SMALL=0;
    both forms against the oracle, forward and adjoint."""
    if small == "multi_kernel":
        monkeypatch.setenv("SLA_SMALL", "0")
    p = SMALL[key]()
    assert p.A.n <= 1024
    x_ref, st, it, _ = oracle.pcg(p.A, p.G, p.eps, p.b, p.rtol, p.maxit)
    w = np.random.default_rng(21).standard_normal(p.A.n)
    lam_ref, g_ref, _, it_a, _ = oracle.adjoint(p.A, p.G, p.eps, x_ref, w, p.rtol, p.maxit)
    say("small system", key, small, p.A.n)
    A, G = handles(p)
    x, info = B.sla_pcg_solve(A, G, p.eps, tdev(p.b), rtol=p.rtol, maxit=p.maxit)
    assert info.status == B.OK and iters_close(info.iterations, it), (info.iterations, it)
    assert rel(host(x), x_ref) <= 1e-8
    gb, gv, ainfo = B.sla_pcg_adjoint(A, G, p.eps, x, tdev(w), rtol=p.rtol, maxit=p.maxit)
    assert iters_close(ainfo.iterations, it_a)
    assert rel(host(gb), lam_ref) <= 1e-7 and rel(host(gv), g_ref) <= 1e-7
    # fp32 storage
    p32 = p.astype("f32")
    A32, G32 = handles(p32, dtype="f32")
    x32, info32 = B.sla_pcg_solve(A32, G32, p.eps, tdev(p32.b), rtol=1e-5, maxit=p.maxit)
    assert info32.status in (B.OK, B.NOT_CONVERGED)
    b64 = p32.b.astype(np.float64)
    res = oracle.spmv(p32.A.astype(np.float64), host(x32)) - b64
    assert np.linalg.norm(res) <= 1e-3 * np.linalg.norm(b64)


def test_small_system_wide_rows_fall_back():
    """Rows wider than the one-workgroup solver keeps in registers take the
    multi-kernel path, with the same results."""
    rng = np.random.default_rng(23)
    A = I.random_spd_csr(900, rng, max_deg=14)
    G = I.spai_factor(A, np.random.default_rng(24))
    b = rng.standard_normal(A.n)
    x_ref, st, it, _ = oracle.pcg(A, G, 3e-3, b, 1e-10, 2000)
    say("small system with wide rows", A.n)
    Ah, Gh = create(A), create(G, transpose=True)
    x, info = B.sla_pcg_solve(Ah, Gh, 3e-3, tdev(b), rtol=1e-10, maxit=2000)
    assert info.status == B.OK and iters_close(info.iterations, it)
    assert rel(host(x), x_ref) <= 1e-8


@pytest.mark.parametrize("every", [1, 5])
def test_profiling_launch_counts(every, monkeypatch):
    """The A-step timing counts one launch per iteration that did work, or
    one per iteration index divisible by the sampling stride."""
    monkeypatch.setenv("SLA_SMALL", "0")
    A = I.poisson2d(37)
    G = I.spai_factor(A, np.random.default_rng(4))
    b = I.spmv_test_vector(2, A.n)
    say("profiling counts, stride", every)
    hA, hG = create(A), create(G, transpose=True)
    B.sla_reset_profile()
    B.sla_set_profiling_stride(every)
    B.sla_set_profiling(["a_step"])
    try:
        _, info = B.sla_pcg_solve(hA, hG, 3e-3, tdev(b), rtol=1e-10, maxit=2000)
    finally:
        B.sla_set_profiling(False)
        B.sla_set_profiling_stride(1)
    n, ms = B.sla_get_profile("a_step")
    assert n == info.iterations // every
    assert ms > 0.0
    with pytest.raises(B.SlaError) as e:
        B.sla_set_profiling_stride(0)
    assert e.value.status == B.ERR_INVALID_ARG


ENGINE_VARIANTS = [{"SLA_SELL16": "0", "SLA_MALL_POLICY": "none"}, {"SLA_MALL_POLICY": "none"},
                   {"SLA_SELL": "0"}, {"SLA_SELL16": "0", "SLA_FUSION": "fused"},
                   {"SLA_SELL": "0", "SLA_FUSION": "fused"},
                   {"SLA_SELL16": "0", "SLA_FUSION": "unfused"}]


@pytest.mark.parametrize("key", ["bsr_elastic_6", "poisson3d_13"])
@pytest.mark.parametrize("env", ENGINE_VARIANTS)
def test_engine_variants(key, env, monkeypatch):
    """Forward and adjoint parity through each engine form the defaults do
    not reach at these sizes: int32 (block) columns in the sliced layouts,
    matrices streamed non-temporally (as when they exceed the Infinity Cache
    budget), the tile / block-row engines without the sliced layout, and the
    iteration form the library would not pick."""
    monkeypatch.setenv("SLA_SMALL", "0")
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    p = problem(key)
    x_ref, st, it, _ = oracle.pcg(p.A, p.G, p.eps, p.b, p.rtol, p.maxit)
    gx_ref = I.loss_grad_weights(p, x_ref)
    lam_ref, gv_ref, st2, it2, _ = oracle.adjoint(p.A, p.G, p.eps, x_ref, gx_ref, p.rtol, p.maxit)
    say("engine variant", key, env)
    A, G = handles(p)
    x, info = B.sla_pcg_solve(A, G, p.eps, tdev(p.b), rtol=p.rtol, maxit=p.maxit)
    assert info.status == B.OK and iters_close(info.iterations, it)
    assert rel(host(x), x_ref) <= 1e-8
    gx = 2.0 * x if p.loss == "sumsq" else tdev(p.w)
    grad_b, grad_vals, ainfo = B.sla_pcg_adjoint(A, G, p.eps, x, gx, rtol=p.rtol, maxit=p.maxit)
    assert ainfo.status == B.OK and iters_close(ainfo.iterations, it2)
    assert rel(host(grad_b), lam_ref) <= 1e-7
    assert rel(host(grad_vals), gv_ref) <= 1e-7


@pytest.mark.parametrize("key", ["poisson3d_13", "heat2d_64", "poisson2d_37", "c2"])
def test_window_engine_bit_identical(key, fusion, monkeypatch):
    """The windowed slice-offset engine (an LDS window of the gathered vector
    serves the slots within 128 rows) solves bit-identically to the plain
    slice-offset engine, on the A steps only (default) and on every step,
    and matches the oracle."""
    if fusion != "auto" and key == "c2":
        pytest.skip("full-size configs run in the library's own choice only")
    p = problem(key)
    monkeypatch.setenv("SLA_SMALL", "0")
    x_ref, _, it_ref, _ = oracle.pcg(p.A, p.G, p.eps, p.b, p.rtol, p.maxit)
    outs = []
    for level in ("0", "1", "2"):
        monkeypatch.setenv("SLA_WIN", level)
        say("window engine", key, fusion, "level", level)
        A, G = handles(p)
        x, info = B.sla_pcg_solve(A, G, p.eps, tdev(p.b), rtol=p.rtol, maxit=p.maxit)
        assert info.status == B.OK
        outs.append((host(x), info.iterations))
    for x, it in outs[1:]:
        assert it == outs[0][1] and np.array_equal(x, outs[0][0])
    assert iters_close(outs[0][1], it_ref) and rel(outs[0][0], x_ref) <= 1e-8
