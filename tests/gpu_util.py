"""Helpers shared by the GPU parity tests (marshalling only)."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from preconditioned_cg_solver_amd import binding as B
from preconditioned_cg_solver_amd import inputs as I

DEV = "cuda:0"


def say(*args):
    """Name the case before a GPU step (and flush), so a failing run names it."""
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def tdev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def torch_dtype(p_or_dtype):
    d = p_or_dtype if isinstance(p_or_dtype, str) else p_or_dtype.dtype
    return torch.float32 if d == "f32" else torch.float64


def np_dtype(dt: str):
    return np.float32 if dt == "f32" else np.float64


def create(M: I.SparseMatrix, transpose=False, validate=True, dtype="f64") -> B.Mat:
    vals = tdev(M.vals.astype(np_dtype(dtype)))
    rp = tdev(M.row_ptr.astype(np.int32))
    ci = tdev(M.col_idx.astype(np.int32))
    if M.block_dim == 1:
        return B.sla_csr_create(rp, ci, vals, build_transpose=transpose, validate=validate)
    return B.sla_bsr_create(rp, ci, vals, block_dim=M.block_dim, build_transpose=transpose,
                            validate=validate)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float64)


def rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def iters_close(k_gpu: int, k_ref: int) -> bool:
    return abs(k_gpu - k_ref) <= max(1, math.ceil(0.02 * k_ref))


def oracle_self_sensitivity(A, G, eps, b, rtol, maxit, seed=0):
    """How far the oracle's own iterate and recursive residual norm move when
    b is perturbed by about one ulp: CG amplifies rounding on ill-conditioned
    systems, so this is the yardstick for comparing two implementations'
    intermediate iterates.  Returns (relative change of x, relative change of
    ||r_k|| / ||b||)."""
    import oracle
    b2 = b * (1.0 + 1e-16 * np.random.default_rng(seed).standard_normal(b.shape))
    x1, _, _, r1 = oracle.pcg(A, G, eps, b, rtol, maxit)
    x2, _, _, r2 = oracle.pcg(A, G, eps, b2, rtol, maxit)
    return rel(x2, x1), abs(r2 - r1) / max(abs(r1), 1e-300)


# Cases that passed through the oracle-spread reading rather than the fixed
# gates; conftest prints them at the end of the run.
FALLBACKS = []


def iters_gate(k_ref: int) -> int:
    """Half-width of the fixed iteration gate: 2% of the oracle's count, at
    least one iteration."""
    return max(1, math.ceil(0.02 * k_ref))


def assert_iterations_match(A, G, eps, b, rtol, maxit, it_g, it_r, strict, what="", rec=None):
    """The GPU's iteration count against the oracle's: within 2% (at least
    1).  Where strict is False (the test matrices beyond the benchmark
    workloads) and that fails, the gate is re-taken against the oracle's own
    spread (oracle_spread) -- but only when that spread is at least as wide as
    the fixed gate, i.e. when rounding alone moves the oracle's stopping
    iteration as far as 2% would allow: then the count must lie within the
    spread, +-1.  Every case that takes this route is printed and recorded
    in FALLBACKS."""
    if iters_close(it_g, it_r):
        return None
    assert not strict, (what, "iterations", it_g, it_r)
    lo, hi, dx = oracle_spread(A, G, eps, b, rtol, maxit)
    r = dict(what=what, it_gpu=it_g, it_ref=it_r, spread=(lo, hi), x_spread=dx)
    if rec:
        r.update(rec)
    assert hi - lo >= iters_gate(it_r), (what, "iterations outside 2% while the oracle's "
                                         "rounding spread is narrower than that", r)
    assert lo - 1 <= it_g <= hi + 1, (what, "iterations outside the oracle's spread", r)
    FALLBACKS.append(r)
    print("[fallback]", r, flush=True)
    return dx


def assert_solve_matches(A, G, eps, b, rtol, maxit, it_g, x_g, it_r, x_r, strict, what=""):
    """The GPU solve against the oracle's: iterations within 2% and x within
    1e-8.  Where strict is False, a gate that fails is re-taken against the
    oracle's own rounding spread, and only when that spread is itself at
    least as wide as the fixed gate (assert_iterations_match): on systems
    whose residual stagnates near rtol the stopping iteration is decided by
    rounding, and any change of summation order or contraction moves it.  x
    may then differ by up to ten times the oracle's own largest change (and
    only if that change exceeds 1e-8)."""
    err = rel(x_g, x_r)
    dx = assert_iterations_match(A, G, eps, b, rtol, maxit, it_g, it_r, strict, what,
                                 dict(x_err=err))
    if err <= 1e-8:
        return
    assert not strict, (what, "x", err)
    if dx is None:
        _, _, dx = oracle_spread(A, G, eps, b, rtol, maxit)
    r = dict(what=what, it_gpu=it_g, it_ref=it_r, x_err=err, x_spread=dx)
    assert dx > 1e-8, (what, "x outside 1e-8 while the oracle's spread is inside it", r)
    assert err <= 10 * dx, (what, "x outside ten times the oracle's spread", r)
    FALLBACKS.append(r)
    print("[fallback]", r, flush=True)


_spread_cache = {}


def oracle_spread(A, G, eps, b, rtol, maxit, nsamp=6):
    """The oracle's own spread under rounding changes: (fewest and most
    iterations, largest relative change of x) over its solves of b and of
    nsamp one-ulp perturbations of b (b (1 + 1e-16 g), g seeded), each by
    the plain build and by the same source built with contracted
    multiply-adds (oracle.load_contracted).  On systems whose residual
    stagnates near rtol the stopping iteration is decided by rounding; this
    is the yardstick for an implementation whose rounding differs."""
    import oracle
    key = (id(A), id(G), float(eps), hash(np.ascontiguousarray(b).tobytes()), float(rtol),
           int(maxit), nsamp)
    if key in _spread_cache:
        return _spread_cache[key]
    libs = (oracle.load(), oracle.load_contracted())
    x0, _, it0, _ = oracle.pcg(A, G, eps, b, rtol, maxit, lib=libs[0])
    its, dx = [it0], 0.0
    for s in range(-1, nsamp):
        b2 = b if s < 0 else b * (1.0 + 1e-16 * np.random.default_rng(s).standard_normal(b.shape))
        for lib in libs:
            if s < 0 and lib is libs[0]:
                continue
            x2, _, it2, _ = oracle.pcg(A, G, eps, b2, rtol, maxit, lib=lib)
            its.append(it2)
            dx = max(dx, rel(x2, x0))
    _spread_cache[key] = (min(its), max(its), dx)
    return _spread_cache[key]


def copy_device_ints(ptr: int, count: int) -> np.ndarray:
    """Copy `count` int32 from a raw device pointer owned by the library."""
    out = torch.empty(count, dtype=torch.int32, device=DEV)
    _memcpy_d2d(out.data_ptr(), ptr, count * 4)
    return out.cpu().numpy()


def copy_device_vals(ptr: int, count: int, dtype=torch.float64) -> np.ndarray:
    out = torch.empty(count, dtype=dtype, device=DEV)
    _memcpy_d2d(out.data_ptr(), ptr, count * out.element_size())
    return out.cpu().numpy()


_hip = None


def _memcpy_d2d(dst: int, src: int, nbytes: int):
    """Device-to-device copy through the HIP runtime torch already loaded."""
    import ctypes
    global _hip
    if _hip is None:
        import os
        libdir = os.path.join(os.path.dirname(torch.__file__), "lib")
        _hip = ctypes.CDLL(os.path.join(libdir, "libamdhip64.so"))
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    torch.cuda.synchronize()
    rc = _hip.hipMemcpy(ctypes.c_void_p(dst), ctypes.c_void_p(src), nbytes, 3)
    assert rc == 0, f"hipMemcpy failed: {rc}"


# Seeded problems shared by the GPU tests, built once per process.
_cache = {}


def problem(key):
    if key not in _cache:
        if key == "c0":
            p = I.make_problem(0)
        elif key == "c1":
            p = I.make_problem(1)
        elif key == "c2":
            p = I.make_problem(2)
        elif key == "c3":
            p = I.make_problem(3)
        elif key == "poisson2d_37":
            p = I.make_problem(0, size=37)
        elif key == "poisson3d_13":
            p = I.make_problem(2, size=13)
        elif key == "bsr_elastic_6":
            p = I.make_problem(3, size=6)
        elif key == "irregular_long_rows":
            A = I.random_spd_csr(12000, np.random.default_rng(8), max_deg=6, long_rows=5,
                                 long_deg=9000)
            G = I.spai_factor(A, np.random.default_rng(9))
            b = np.random.default_rng(10).standard_normal(A.n)
            p = I.Problem("irregular_long_rows", -1, A, G, b, 3e-3, 1e-10, 5000, "dot",
                          np.random.default_rng(11).standard_normal(A.n))
        elif key == "powerlaw_20k":
            p = I.make_problem(4, size=20000)
        elif key == "heat2d_64":
            p = I.make_problem(1, size=64)
        elif key == "poisson3d_92":
            p = I.make_problem(2, size=92)
        else:
            raise KeyError(key)
        _cache[key] = p
    return _cache[key]
