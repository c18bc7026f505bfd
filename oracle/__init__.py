"""CPU parity oracle (test infrastructure only).

Thin ctypes wrapper over ``oracle.c`` (plain fp64 C, built with gcc).  Only the
tests, the smoke check and the benchmark's CPU-baseline leg use this package;
the product path (the HIP library and its binding) never imports it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
# The same source built with multiply-adds contracted to FMA instructions.
# Not a second oracle: the parity tests use it only to measure how far the
# oracle's own stopping iteration moves under rounding changes of the kind a
# GPU makes (fused multiply-adds).
LIB_CONTRACTED = os.path.join(HERE, "liboracle_contracted.so")
CONTRACTED_FLAGS = ("-mfma", "-ffp-contract=fast")
# The same source with rows longer than 2,048 entries summed in 4,096-entry
# chunks (ORC_ROW_CHUNK in oracle.c): likewise only a yardstick for how far
# the stopping iteration moves with the summation order of very long rows.
LIB_CHUNKED = os.path.join(HERE, "liboracle_chunked.so")
CHUNKED_FLAGS = ("-DORC_ROW_CHUNK=4096",)

OK, NOT_CONVERGED, ERR_ARG, ERR_BREAKDOWN, ERR_NONFINITE, ERR_NOMEM = 0, 1, -1, -3, -4, -6

_lock = threading.Lock()
_lib = None
_lib_contracted = None
_lib_chunked = None


def build(src: str = SRC, out: str = LIB, extra_flags: Tuple[str, ...] = ()) -> str:
    """Compile the oracle with gcc (-O2, no FP contraction, OpenMP over rows)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared", "-std=c11", *extra_flags, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: Optional[str] = None):
    global _lib
    with _lock:
        if path is not None:
            return _bind(ctypes.CDLL(path))
        if _lib is None:
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build()
            _lib = _bind(ctypes.CDLL(LIB))
        return _lib


def load_contracted():
    """The oracle built with contracted multiply-adds (see LIB_CONTRACTED)."""
    global _lib_contracted
    with _lock:
        if _lib_contracted is None:
            if (not os.path.exists(LIB_CONTRACTED)
                    or os.path.getmtime(LIB_CONTRACTED) < os.path.getmtime(SRC)):
                build(out=LIB_CONTRACTED, extra_flags=CONTRACTED_FLAGS)
            _lib_contracted = _bind(ctypes.CDLL(LIB_CONTRACTED))
        return _lib_contracted


def load_chunked():
    """The oracle built with chunked sums of very long rows (see LIB_CHUNKED)."""
    global _lib_chunked
    with _lock:
        if _lib_chunked is None:
            if (not os.path.exists(LIB_CHUNKED)
                    or os.path.getmtime(LIB_CHUNKED) < os.path.getmtime(SRC)):
                build(out=LIB_CHUNKED, extra_flags=CHUNKED_FLAGS)
            _lib_chunked = _bind(ctypes.CDLL(LIB_CHUNKED))
        return _lib_chunked


def _bind(lib):
    i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
    lib.orc_spmv.argtypes = [i64, ctypes.c_int, vp, vp, vp, vp, vp]
    lib.orc_spmv.restype = None
    lib.orc_transpose.argtypes = [i64, ctypes.c_int, vp, vp, vp, vp, vp, vp]
    lib.orc_transpose.restype = ctypes.c_int
    lib.orc_dot.argtypes = [i64, vp, vp]
    lib.orc_dot.restype = dbl
    lib.orc_precond_apply.argtypes = [i64, ctypes.c_int, vp, vp, vp, dbl, vp, vp]
    lib.orc_precond_apply.restype = ctypes.c_int
    lib.orc_pcg.argtypes = [i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, dbl, vp, vp, dbl, i32,
                            ctypes.POINTER(i32), ctypes.POINTER(dbl)]
    lib.orc_pcg.restype = ctypes.c_int
    lib.orc_adjoint.argtypes = [i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, dbl, vp, vp, vp, vp,
                                dbl, i32, ctypes.POINTER(i32), ctypes.POINTER(dbl)]
    lib.orc_adjoint.restype = ctypes.c_int
    lib.orc_pattern_grad.argtypes = [i64, ctypes.c_int, vp, vp, vp, vp, vp]
    lib.orc_pattern_grad.restype = None
    lib.orc_pcg_history.argtypes = [i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, dbl, vp, vp, dbl,
                                    i32, ctypes.POINTER(i32), ctypes.POINTER(dbl), vp, vp, i32]
    lib.orc_pcg_history.restype = ctypes.c_int
    lib.orc_lanczos_tridiag.argtypes = [vp, vp, i32, vp, vp]
    lib.orc_lanczos_tridiag.restype = ctypes.c_int
    lib.orc_sai_loss.argtypes = [i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, dbl, vp, i32, dbl, vp]
    lib.orc_sai_loss.restype = ctypes.c_int
    lib.orc_pcg_multi.argtypes = [i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, dbl, vp, vp, i32, dbl,
                                  i32, vp, vp, vp]
    lib.orc_pcg_multi.restype = ctypes.c_int
    lib.orc_adjoint_multi.argtypes = [i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, dbl, vp, vp, vp,
                                      vp, i32, dbl, i32, vp, vp, vp]
    lib.orc_adjoint_multi.restype = ctypes.c_int
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_set_num_threads.argtypes = [ctypes.c_int]
    lib.orc_set_num_threads.restype = None
    lib.orc_dot_block.argtypes = []
    lib.orc_dot_block.restype = ctypes.c_int
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _mat(M):
    return (_c(M.row_ptr, np.int32), _c(M.col_idx, np.int32), _c(M.vals, np.float64))


def num_threads(lib=None) -> int:
    return int((lib or load()).orc_num_threads())


def set_num_threads(t: int, lib=None) -> None:
    """Threads of the oracle's OpenMP loops for the calling thread's later
    calls (timing only: results do not depend on it)."""
    (lib or load()).orc_set_num_threads(int(t))


def spmv(M, x: np.ndarray, lib=None) -> np.ndarray:
    """y = M x (M a SparseMatrix from the inputs module)."""
    lib = lib or load()
    rp, ci, v = _mat(M)
    x = _c(x, np.float64)
    y = np.empty(M.n, dtype=np.float64)
    lib.orc_spmv(M.n_block_rows, M.block_dim, _p(rp), _p(ci), _p(v), _p(x), _p(y))
    return y


def transpose(M, lib=None):
    """Explicit transpose (row_ptr, col_idx, vals) of a square CSR/BSR matrix."""
    lib = lib or load()
    rp, ci, v = _mat(M)
    trp = np.empty_like(rp)
    tci = np.empty_like(ci)
    tv = np.empty_like(v)
    st = lib.orc_transpose(M.n_block_rows, M.block_dim, _p(rp), _p(ci), _p(v), _p(trp),
                           _p(tci), _p(tv))
    if st != OK:
        raise MemoryError("oracle transpose failed")
    return trp, tci, tv


def dot(a: np.ndarray, b: np.ndarray, lib=None) -> float:
    lib = lib or load()
    a = _c(a, np.float64)
    b = _c(b, np.float64)
    return float(lib.orc_dot(a.shape[0], _p(a), _p(b)))


def precond_apply(G, eps: float, r: np.ndarray, lib=None) -> np.ndarray:
    """z = (G G^T + eps I) r."""
    lib = lib or load()
    rp, ci, v = _mat(G)
    r = _c(r, np.float64)
    z = np.empty(G.n, dtype=np.float64)
    st = lib.orc_precond_apply(G.n_block_rows, G.block_dim, _p(rp), _p(ci), _p(v), eps, _p(r),
                               _p(z))
    if st != OK:
        raise MemoryError("oracle precond_apply failed")
    return z


def pcg(A, G, eps: float, b: np.ndarray, rtol: float, maxit: int, lib=None):
    """Returns (x, status, iterations, recursive relative residual)."""
    lib = lib or load()
    arp, aci, av = _mat(A)
    grp, gci, gv = _mat(G)
    b = _c(b, np.float64)
    x = np.empty(A.n, dtype=np.float64)
    it = ctypes.c_int32(0)
    rr = ctypes.c_double(0.0)
    st = lib.orc_pcg(A.n_block_rows, A.block_dim, _p(arp), _p(aci), _p(av), _p(grp), _p(gci),
                     _p(gv), float(eps), _p(b), _p(x), float(rtol), int(maxit),
                     ctypes.byref(it), ctypes.byref(rr))
    return x, int(st), int(it.value), float(rr.value)


def pcg_history(A, G, eps: float, b: np.ndarray, rtol: float, maxit: int, lib=None):
    """pcg that also returns the CG coefficients: (x, status, iterations, relres,
    alpha[0:iterations], beta[0:iterations-1]) with beta_k = rho_k / rho_{k-1}."""
    lib = lib or load()
    arp, aci, av = _mat(A)
    grp, gci, gv = _mat(G)
    b = _c(b, np.float64)
    x = np.empty(A.n, dtype=np.float64)
    m = max(int(maxit), 1)
    ha = np.zeros(m, dtype=np.float64)
    hb = np.zeros(m, dtype=np.float64)
    it = ctypes.c_int32(0)
    rr = ctypes.c_double(0.0)
    st = lib.orc_pcg_history(A.n_block_rows, A.block_dim, _p(arp), _p(aci), _p(av), _p(grp),
                             _p(gci), _p(gv), float(eps), _p(b), _p(x), float(rtol), int(maxit),
                             ctypes.byref(it), ctypes.byref(rr), _p(ha), _p(hb), m)
    k = int(it.value)
    return x, int(st), k, float(rr.value), ha[:k].copy(), hb[:max(k - 1, 0)].copy()


def lanczos_tridiag(alpha: np.ndarray, beta: np.ndarray, lib=None):
    """(diagonal, off-diagonal) of the Lanczos tridiagonal built from CG's
    alpha_1..k and beta_1..k-1."""
    lib = lib or load()
    a = _c(alpha, np.float64)
    k = a.shape[0]
    b = _c(beta, np.float64) if k > 1 else np.zeros(1)
    d = np.empty(max(k, 1), dtype=np.float64)
    e = np.empty(max(k - 1, 1), dtype=np.float64)
    st = lib.orc_lanczos_tridiag(_p(a), _p(b), k, _p(d), _p(e))
    if st != OK:
        raise ValueError("lanczos_tridiag: need k >= 1, alpha > 0, beta >= 0")
    return d[:k], e[:k - 1]


def ritz_values(alpha: np.ndarray, beta: np.ndarray, lib=None) -> np.ndarray:
    """Eigenvalues (ascending) of the Lanczos tridiagonal: Ritz values of M^-1 A
    (scipy's symmetric tridiagonal eigensolver is the library step)."""
    from scipy.linalg import eigvalsh_tridiagonal
    d, e = lanczos_tridiag(alpha, beta, lib)
    if d.shape[0] == 1:
        return d.copy()
    return eigvalsh_tridiagonal(d, e)


def sai_loss(A, G, eps: float, W: np.ndarray, scale: float, lib=None) -> np.ndarray:
    """Per-probe || A M^-1 w_j / scale - w_j ||^2 for the columns w_j of W (n x m)."""
    lib = lib or load()
    arp, aci, av = _mat(A)
    grp, gci, gv = _mat(G)
    W = np.asarray(W, dtype=np.float64)
    m = W.shape[1]
    w = np.ascontiguousarray(W.T)  # probe j contiguous at j * n
    out = np.empty(max(m, 1), dtype=np.float64)
    st = lib.orc_sai_loss(A.n_block_rows, A.block_dim, _p(arp), _p(aci), _p(av), _p(grp),
                          _p(gci), _p(gv), float(eps), _p(w), m, float(scale), _p(out))
    if st != OK:
        raise ValueError("sai_loss: bad argument")
    return out[:m]


def dense_spectrum(A, G, eps: float) -> np.ndarray:
    """All eigenvalues (ascending) of M^-1 A with M^-1 = G G^T + eps I, for small
    matrices: M^-1 = L L^T (Cholesky) makes M^-1 A similar to L^T A L."""
    Ad = A.to_dense()
    Gd = G.to_dense()
    Minv = Gd @ Gd.T + eps * np.eye(A.n)
    L = np.linalg.cholesky(Minv)
    S = L.T @ Ad @ L
    return np.linalg.eigvalsh(0.5 * (S + S.T))


def kaporin_number(eigs: np.ndarray) -> float:
    """Kaporin's condition number of an SPD operator: the arithmetic mean of its
    eigenvalues over their geometric mean (1 for a multiple of I)."""
    e = np.asarray(eigs, dtype=np.float64)
    return float(np.mean(e) / np.exp(np.mean(np.log(e))))


def pcg_multi(A, G, eps: float, B: np.ndarray, rtol: float, maxit: int, lib=None):
    """k right-hand sides (columns of the n x k array B): returns (X n x k,
    overall status, per-column iterations, relres, status)."""
    lib = lib or load()
    arp, aci, av = _mat(A)
    grp, gci, gv = _mat(G)
    B = _c(B, np.float64)
    k = B.shape[1]
    X = np.empty_like(B)
    it = np.zeros(k, dtype=np.int32)
    rr = np.zeros(k, dtype=np.float64)
    sts = np.zeros(k, dtype=np.int32)
    st = lib.orc_pcg_multi(A.n_block_rows, A.block_dim, _p(arp), _p(aci), _p(av), _p(grp),
                           _p(gci), _p(gv), float(eps), _p(B), _p(X), k, float(rtol), int(maxit),
                           _p(it), _p(rr), _p(sts))
    return X, int(st), it, rr, sts


def adjoint_multi(A, G, eps: float, X: np.ndarray, GX: np.ndarray, rtol: float, maxit: int,
                  lib=None):
    """Adjoint of k solves sharing A: returns (Lambda = dL/dB (n x k), dL/dvals
    summed over the solves, overall status, per-column iterations, relres, status)."""
    lib = lib or load()
    arp, aci, av = _mat(A)
    grp, gci, gv = _mat(G)
    X = _c(X, np.float64)
    GX = _c(GX, np.float64)
    k = X.shape[1]
    lam = np.empty_like(X)
    gval = np.empty(av.shape[0], dtype=np.float64)
    it = np.zeros(k, dtype=np.int32)
    rr = np.zeros(k, dtype=np.float64)
    sts = np.zeros(k, dtype=np.int32)
    st = lib.orc_adjoint_multi(A.n_block_rows, A.block_dim, _p(arp), _p(aci), _p(av), _p(grp),
                               _p(gci), _p(gv), float(eps), _p(X), _p(GX), _p(lam), _p(gval), k,
                               float(rtol), int(maxit), _p(it), _p(rr), _p(sts))
    return lam, gval, int(st), it, rr, sts


def pattern_grad(A, lam: np.ndarray, x: np.ndarray, lib=None) -> np.ndarray:
    """dL/dvals[k] = -lam_row(k) * x_col(k) in A's storage order."""
    lib = lib or load()
    arp, aci, _ = _mat(A)
    lam = _c(lam, np.float64)
    x = _c(x, np.float64)
    g = np.empty(A.nnz, dtype=np.float64)
    lib.orc_pattern_grad(A.n_block_rows, A.block_dim, _p(arp), _p(aci), _p(lam), _p(x), _p(g))
    return g


def adjoint(A, G, eps: float, x: np.ndarray, gx: np.ndarray, rtol: float, maxit: int, lib=None):
    """Returns (lambda = dL/db, dL/dvals in A's storage order, status, iterations, relres)."""
    lib = lib or load()
    arp, aci, av = _mat(A)
    grp, gci, gv = _mat(G)
    x = _c(x, np.float64)
    gx = _c(gx, np.float64)
    lam = np.empty(A.n, dtype=np.float64)
    gval = np.empty(av.shape[0], dtype=np.float64)
    it = ctypes.c_int32(0)
    rr = ctypes.c_double(0.0)
    st = lib.orc_adjoint(A.n_block_rows, A.block_dim, _p(arp), _p(aci), _p(av), _p(grp),
                         _p(gci), _p(gv), float(eps), _p(x), _p(gx), _p(lam), _p(gval),
                         float(rtol), int(maxit), ctypes.byref(it), ctypes.byref(rr))
    return lam, gval, int(st), int(it.value), float(rr.value)
