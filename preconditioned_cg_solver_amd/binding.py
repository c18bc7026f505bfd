"""ctypes binding of ``libsla.so`` (the C ABI in ``include/sla.h``).

Argument marshalling only: every numerical step runs in the library's HIP
kernels.  Torch tensors supply device memory and the current HIP stream.
torch is imported before the library is loaded so that ``libsla.so`` binds to
the same HIP runtime instance as torch (both carry the soname
``libamdhip64.so.7``).  There is no CPU fallback: if the library is missing or
no GPU is present, the calls raise.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import threading
from typing import Optional, Tuple

import torch  # noqa: F401  (must precede loading libsla.so, see above)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsla.so")

SLA_F64, SLA_F32 = 0, 1
SLA_BUILD_TRANSPOSE, SLA_VALIDATE = 1, 2
STATUS = {0: "SLA_OK", 1: "SLA_NOT_CONVERGED", -1: "SLA_ERR_INVALID_ARG", -2: "SLA_ERR_UNSUPPORTED",
          -3: "SLA_ERR_BREAKDOWN", -4: "SLA_ERR_NONFINITE", -5: "SLA_ERR_HIP", -6: "SLA_ERR_OOM"}
OK, NOT_CONVERGED = 0, 1
ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_BREAKDOWN, ERR_NONFINITE, ERR_HIP, ERR_OOM = -1, -2, -3, -4, -5, -6
PROFILE_CLASSES = {"a_step": 0, "gt_step": 1, "g_step": 2, "spmv": 3}


class SlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class SolveInfo(ctypes.Structure):
    _fields_ = [("iterations", ctypes.c_int32), ("converged", ctypes.c_int32),
                ("rel_residual", ctypes.c_double), ("bnorm", ctypes.c_double)]


_lib = None
_lock = threading.Lock()


def lib_path() -> str:
    """libsla.so, or with SLA_DEBUG=1 the bounds-checking build libsla_debug.so."""
    if os.environ.get("SLA_DEBUG") == "1":
        return os.path.join(PKG, "libsla_debug.so")
    return LIB_PATH


def lib():
    """Load the library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            path = lib_path()
            if not os.path.exists(path):
                raise ImportError(f"{path} is missing: build it with "
                                  "preconditioned_cg_solver_amd.build.build()")
            _lib = _declare(ctypes.CDLL(path))
        return _lib


def _declare(L):
    vp, i32, i64, u32, dbl, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                  ctypes.c_double, ctypes.c_size_t)
    st = ctypes.c_int
    sig = {
        "sla_csr_create": ([ctypes.POINTER(vp), i64, i64, vp, vp, vp, ctypes.c_int, u32, vp], st),
        "sla_bsr_create": ([ctypes.POINTER(vp), i64, i64, i32, vp, vp, vp, ctypes.c_int, u32, vp], st),
        "sla_mat_destroy": ([vp], st),
        "sla_mat_info": ([vp, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i32),
                          ctypes.POINTER(i32)], st),
        "sla_mat_transpose_arrays": ([vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                      ctypes.POINTER(vp)], st),
        "sla_mat_tiling": ([vp, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)], st),
        "sla_mat_reordered": ([vp, ctypes.POINTER(i32)], st),
        "sla_spmv": ([vp, vp, vp, vp], st),
        "sla_spmv_t": ([vp, vp, vp, vp], st),
        "sla_pcg_workspace_size": ([vp, ctypes.POINTER(sz)], st),
        "sla_precond_apply": ([vp, dbl, vp, vp, vp, sz, vp], st),
        "sla_pcg_solve": ([vp, vp, dbl, vp, vp, dbl, i32, vp, sz, vp, ctypes.POINTER(SolveInfo)],
                          st),
        "sla_pcg_adjoint": ([vp, vp, dbl, vp, vp, vp, vp, dbl, i32, vp, sz, vp,
                             ctypes.POINTER(SolveInfo)], st),
        "sla_spmm": ([vp, vp, vp, i32, vp], st),
        "sla_spmm_t": ([vp, vp, vp, i32, vp], st),
        "sla_pcg_workspace_size_multi": ([vp, i32, ctypes.POINTER(sz)], st),
        "sla_pcg_solve_multi": ([vp, vp, dbl, vp, vp, i32, dbl, i32, vp, sz, vp,
                                 ctypes.POINTER(SolveInfo), ctypes.POINTER(ctypes.c_int)], st),
        "sla_pcg_adjoint_multi": ([vp, vp, dbl, vp, vp, vp, vp, i32, dbl, i32, vp, sz, vp,
                                   ctypes.POINTER(SolveInfo), ctypes.POINTER(ctypes.c_int)], st),
        "sla_lanczos_extremes": ([vp, vp, i32, ctypes.POINTER(dbl), ctypes.POINTER(dbl)], st),
        "sla_sai_loss": ([vp, vp, dbl, vp, i32, dbl, vp, sz, vp, vp], st),
        "sla_pcg_solve_history": ([vp, vp, dbl, vp, vp, dbl, i32, vp, sz, vp, vp, i32, vp,
                                   ctypes.POINTER(SolveInfo)], st),
        "sla_pattern_grad": ([vp, vp, vp, vp, vp], st),
        "sla_init": ([], st),
        "sla_pcg_solve_noalloc": ([vp, vp, dbl, vp, vp, dbl, i32, vp, ctypes.POINTER(SolveInfo)],
                                  st),
        "sla_status_string": ([st], ctypes.c_char_p),
        "sla_last_error": ([], ctypes.c_char_p),
        "sla_set_profiling": ([i32], st),
        "sla_set_profiling_stride": ([i32], st),
        "sla_get_profile": ([i32, ctypes.POINTER(i64), ctypes.POINTER(dbl)], st),
        "sla_reset_profile": ([], st),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


def _check(status: int, allow=(OK,)) -> int:
    if status in allow:
        return status
    msg = lib().sla_last_error().decode(errors="replace")
    raise SlaError(status, msg)


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream) if hasattr(stream, "cuda_stream") else stream


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _vec(t: torch.Tensor, A: "Mat", numel: int, name: str):
    """Pointer of a vector argument of a call on A: a contiguous tensor on A's
    device, in A's dtype, with exactly `numel` elements (the library reads
    and writes that many from the raw pointer and cannot check it)."""
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != A.dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, the matrix has {A.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if torch.device(t.device) != torch.device(A.device):
        raise ValueError(f"{name} is on {t.device}, the matrix on {A.device}")
    return ctypes.c_void_p(t.data_ptr())


def _work(work: torch.Tensor, A: "Mat"):
    """(pointer, size in bytes) of a workspace tensor on A's device."""
    if not getattr(work, "is_cuda", False) or not work.is_contiguous():
        raise ValueError("the workspace must be a contiguous GPU tensor")
    if torch.device(work.device) != torch.device(A.device):
        raise ValueError(f"the workspace is on {work.device}, the matrix on {A.device}")
    return ctypes.c_void_p(work.data_ptr()), work.numel() * work.element_size()


def _pair(A: "Mat", G: "Mat"):
    if A.n != G.n or A.dtype != G.dtype or A.block_dim != G.block_dim:
        raise ValueError("A and G differ in size, block size or dtype")


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float64:
        return SLA_F64
    if dt == torch.float32:
        return SLA_F32
    raise ValueError(f"unsupported dtype {dt}")


class Mat:
    """A library matrix handle; keeps the borrowed tensors alive."""

    def __init__(self, handle, keep, n, nnz, block_dim, dtype):
        self.handle = handle
        self._keep = keep
        self.n, self.nnz, self.block_dim, self.dtype = n, nnz, block_dim, dtype

    def destroy(self):
        if self.handle:
            lib().sla_mat_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    @property
    def device(self):
        return self._keep[0].device


def sla_mat_destroy(A: Mat) -> None:
    A.destroy()


def sla_mat_info(A: Mat) -> Tuple[int, int, int, int]:
    """(n, nnz, block_dim, dtype code) as the library records them."""
    n, nnz = ctypes.c_int64(), ctypes.c_int64()
    bd, dt = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().sla_mat_info(A.handle, ctypes.byref(n), ctypes.byref(nnz), ctypes.byref(bd),
                              ctypes.byref(dt)))
    return n.value, nnz.value, bd.value, dt.value


def sla_last_error() -> str:
    return lib().sla_last_error().decode(errors="replace")


def sla_csr_create(row_ptr: torch.Tensor, col_idx: torch.Tensor, vals: torch.Tensor,
                   build_transpose: bool = False, validate: bool = False, stream=None) -> Mat:
    n = row_ptr.numel() - 1
    nnz = col_idx.numel()
    for t, want in ((row_ptr, torch.int32), (col_idx, torch.int32)):
        if t.dtype != want:
            raise ValueError("index arrays must be int32")
    h = ctypes.c_void_p()
    flags = (SLA_BUILD_TRANSPOSE if build_transpose else 0) | (SLA_VALIDATE if validate else 0)
    _check(lib().sla_csr_create(ctypes.byref(h), n, nnz, _ptr(row_ptr), _ptr(col_idx), _ptr(vals),
                                _dtype_code(vals.dtype), flags, _stream(stream)))
    return Mat(h, (row_ptr, col_idx, vals), n, nnz, 1, vals.dtype)


def sla_bsr_create(brow_ptr: torch.Tensor, bcol_idx: torch.Tensor, bvals: torch.Tensor,
                   block_dim: int = 3, build_transpose: bool = False, validate: bool = False,
                   stream=None) -> Mat:
    nbr = brow_ptr.numel() - 1
    nnzb = bcol_idx.numel()
    if bvals.numel() != nnzb * block_dim * block_dim:
        raise ValueError("bvals must hold nnzb * block_dim^2 values")
    h = ctypes.c_void_p()
    flags = (SLA_BUILD_TRANSPOSE if build_transpose else 0) | (SLA_VALIDATE if validate else 0)
    _check(lib().sla_bsr_create(ctypes.byref(h), nbr, nnzb, block_dim, _ptr(brow_ptr),
                                _ptr(bcol_idx), _ptr(bvals), _dtype_code(bvals.dtype), flags,
                                _stream(stream)))
    return Mat(h, (brow_ptr, bcol_idx, bvals), nbr * block_dim, nnzb * block_dim ** 2, block_dim,
               bvals.dtype)


def sla_mat_tiling(A: Mat, transpose: bool = False) -> Tuple[int, int]:
    nt, nl = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().sla_mat_tiling(A.handle, int(transpose), ctypes.byref(nt), ctypes.byref(nl)))
    return nt.value, nl.value


def sla_mat_reordered(A: Mat) -> bool:
    """True when the solves with A run on its locality ordering."""
    r = ctypes.c_int32()
    _check(lib().sla_mat_reordered(A.handle, ctypes.byref(r)))
    return bool(r.value)


def sla_mat_transpose_arrays(A: Mat):
    """Raw device pointers (row_ptr, col_idx, vals) of the owned transpose."""
    rp, ci, v = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
    _check(lib().sla_mat_transpose_arrays(A.handle, ctypes.byref(rp), ctypes.byref(ci),
                                          ctypes.byref(v)))
    return rp.value, ci.value, v.value


def sla_spmv(A: Mat, x: torch.Tensor, y: Optional[torch.Tensor] = None, stream=None,
             transpose: bool = False) -> torch.Tensor:
    px = _vec(x, A, A.n, "x")
    if y is None:
        y = torch.empty(A.n, dtype=A.dtype, device=x.device)
    py = _vec(y, A, A.n, "y")
    f = lib().sla_spmv_t if transpose else lib().sla_spmv
    _check(f(A.handle, px, py, _stream(stream)))
    return y


def sla_spmv_t(A: Mat, x: torch.Tensor, y: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """y = A^T x (the handle must carry its transpose)."""
    return sla_spmv(A, x, y, stream, transpose=True)


def sla_pcg_workspace_size(A: Mat) -> int:
    b = ctypes.c_size_t()
    _check(lib().sla_pcg_workspace_size(A.handle, ctypes.byref(b)))
    return b.value


def workspace(A: Mat, device=None) -> torch.Tensor:
    nbytes = sla_pcg_workspace_size(A)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device or A.device)


def sla_precond_apply(G: Mat, eps: float, r: torch.Tensor, z: Optional[torch.Tensor] = None,
                      work: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    pr = _vec(r, G, G.n, "r")
    if z is None:
        z = torch.empty_like(r)
    pz = _vec(z, G, G.n, "z")
    if work is None:
        work = workspace(G, r.device)
    pw, nw = _work(work, G)
    _check(lib().sla_precond_apply(G.handle, float(eps), pr, pz, pw, nw, _stream(stream)))
    return z


@dataclasses.dataclass
class Info:
    status: int
    iterations: int
    converged: bool
    rel_residual: float
    bnorm: float


def _info(status, si: SolveInfo) -> Info:
    return Info(status, si.iterations, bool(si.converged), si.rel_residual, si.bnorm)


def sla_pcg_solve(A: Mat, G: Mat, eps: float, b: torch.Tensor, x: Optional[torch.Tensor] = None,
                  rtol: float = 1e-10, maxit: int = 1000, work: Optional[torch.Tensor] = None,
                  stream=None, raise_on_error: bool = True) -> Tuple[torch.Tensor, Info]:
    _pair(A, G)
    pb = _vec(b, A, A.n, "b")
    if x is None:
        x = torch.empty_like(b)
    px = _vec(x, A, A.n, "x")
    if work is None:
        work = workspace(A, b.device)
    pw, nw = _work(work, A)
    si = SolveInfo()
    st = lib().sla_pcg_solve(A.handle, G.handle, float(eps), pb, px, float(rtol), int(maxit), pw,
                             nw, _stream(stream), ctypes.byref(si))
    if raise_on_error:
        _check(st, allow=(OK, NOT_CONVERGED))
    return x, _info(st, si)


def sla_init() -> None:
    """Prepare the current device for sla_pcg_solve_noalloc (resolves the
    library's fixed scratch and reserves a polling record; may allocate)."""
    _check(lib().sla_init())


def sla_pcg_solve_noalloc(A: Mat, G: Mat, eps: float, b: torch.Tensor, x: torch.Tensor,
                          rtol: float = 1e-10, maxit: int = 1000, stream=None,
                          raise_on_error: bool = True) -> Info:
    """sla_pcg_solve with the library's fixed scratch as workspace: allocates
    nothing (x is the caller's output tensor).  Needs sla_init() first."""
    _pair(A, G)
    pb = _vec(b, A, A.n, "b")
    px = _vec(x, A, A.n, "x")
    si = SolveInfo()
    st = lib().sla_pcg_solve_noalloc(A.handle, G.handle, float(eps), pb, px, float(rtol),
                                     int(maxit), _stream(stream), ctypes.byref(si))
    if raise_on_error:
        _check(st, allow=(OK, NOT_CONVERGED))
    return _info(st, si)


def sla_pcg_solve_history(A: Mat, G: Mat, eps: float, b: torch.Tensor,
                          x: Optional[torch.Tensor] = None, rtol: float = 1e-10,
                          maxit: int = 1000, work: Optional[torch.Tensor] = None, stream=None,
                          raise_on_error: bool = True):
    """sla_pcg_solve that also returns the CG coefficients alpha_k (k = 1..iters)
    and beta_k = rho_k / rho_{k-1} (k = 1..iters-1) as CPU float64 tensors."""
    _pair(A, G)
    pb = _vec(b, A, A.n, "b")
    if x is None:
        x = torch.empty_like(b)
    px = _vec(x, A, A.n, "x")
    if work is None:
        work = workspace(A, b.device)
    pw, nw = _work(work, A)
    hist_a = torch.zeros(max(maxit, 1), dtype=torch.float64, device=b.device)
    hist_b = torch.zeros(max(maxit, 1), dtype=torch.float64, device=b.device)
    si = SolveInfo()
    st = lib().sla_pcg_solve_history(A.handle, G.handle, float(eps), pb, px, float(rtol),
                                     int(maxit), pw, nw, _ptr(hist_a), _ptr(hist_b), int(maxit),
                                     _stream(stream), ctypes.byref(si))
    if raise_on_error:
        _check(st, allow=(OK, NOT_CONVERGED))
    k = si.iterations
    return x, _info(st, si), hist_a[:k].cpu(), hist_b[:max(k - 1, 0)].cpu()


def sla_lanczos_extremes(alpha, beta):
    """(lmin, lmax) of the Lanczos tridiagonal from CG's alpha_1..k, beta_1..k-1."""
    a = [float(v) for v in alpha]
    b = [float(v) for v in beta] or [0.0]
    ha = (ctypes.c_double * max(len(a), 1))(*a)
    hb = (ctypes.c_double * len(b))(*b)
    lo, hi = ctypes.c_double(0.0), ctypes.c_double(0.0)
    st = lib().sla_lanczos_extremes(ha, hb, len(a), ctypes.byref(lo), ctypes.byref(hi))
    _check(st)
    return lo.value, hi.value


def sla_sai_loss(A: Mat, G: Mat, eps: float, probes: torch.Tensor, scale: float,
                 work: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Per-probe || A M^-1 w_j / scale - w_j ||^2 for the columns w_j of the
    (n, m) device tensor `probes` (float64 device tensor of length m)."""
    _pair(A, G)
    if probes.dim() != 2 or probes.shape[0] != A.n:
        raise ValueError(f"probes must be ({A.n}, m)")
    n, m = probes.shape
    pt = probes.t().contiguous()  # probe j contiguous at j * n
    pp = _vec(pt, A, n * m, "probes")
    if work is None:
        nb = max(sla_pcg_workspace_size(A), sla_pcg_workspace_size(G), 1)
        work = torch.empty(nb, dtype=torch.uint8, device=probes.device)
    pw, nw = _work(work, A)
    out = torch.empty(max(m, 1), dtype=torch.float64, device=probes.device)
    st = lib().sla_sai_loss(A.handle, G.handle, float(eps), pp, int(m), float(scale), pw, nw,
                            _ptr(out), _stream(stream))
    _check(st)
    return out[:m]


def sla_pcg_adjoint(A: Mat, G: Mat, eps: float, x: torch.Tensor, grad_x: torch.Tensor,
                    rtol: float = 1e-10, maxit: int = 1000, grad_b: Optional[torch.Tensor] = None,
                    grad_vals: Optional[torch.Tensor] = None, work: Optional[torch.Tensor] = None,
                    stream=None, raise_on_error: bool = True):
    _pair(A, G)
    px = _vec(x, A, A.n, "x")
    pgx = _vec(grad_x, A, A.n, "grad_x")
    if grad_b is None:
        grad_b = torch.empty_like(x)
    pgb = _vec(grad_b, A, A.n, "grad_b")
    if grad_vals is None:
        grad_vals = torch.empty(A.nnz, dtype=A.dtype, device=x.device)
    pgv = _vec(grad_vals, A, A.nnz, "grad_vals")
    if work is None:
        work = workspace(A, x.device)
    pw, nw = _work(work, A)
    si = SolveInfo()
    st = lib().sla_pcg_adjoint(A.handle, G.handle, float(eps), px, pgx, pgb, pgv, float(rtol),
                               int(maxit), pw, nw, _stream(stream), ctypes.byref(si))
    if raise_on_error:
        _check(st, allow=(OK, NOT_CONVERGED))
    return grad_b, grad_vals, _info(st, si)


# ----- several right-hand sides (n x k row-major device tensors) -----

def _cols(t: torch.Tensor, A: "Mat" = None) -> int:
    if t.dim() != 2 or not t.is_contiguous():
        raise ValueError("expected a contiguous (n, k) tensor")
    if A is not None and t.shape[0] != A.n:
        raise ValueError(f"expected {A.n} rows, got {t.shape[0]}")
    return t.shape[1]


def _block(t: torch.Tensor, A: "Mat", k: int, name: str):
    if t.dim() != 2 or tuple(t.shape) != (A.n, k):
        raise ValueError(f"{name} must be ({A.n}, {k}), got {tuple(t.shape)}")
    return _vec(t, A, A.n * k, name)


def sla_spmm(A: Mat, X: torch.Tensor, Y: Optional[torch.Tensor] = None,
             stream=None) -> torch.Tensor:
    """Y = A X for the k columns of the (n, k) tensor X."""
    k = _cols(X, A)
    px = _block(X, A, k, "X")
    if Y is None:
        Y = torch.empty_like(X)
    py = _block(Y, A, k, "Y")
    _check(lib().sla_spmm(A.handle, px, py, k, _stream(stream)))
    return Y


def sla_spmm_t(A: Mat, X: torch.Tensor, Y: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    k = _cols(X, A)
    px = _block(X, A, k, "X")
    if Y is None:
        Y = torch.empty_like(X)
    py = _block(Y, A, k, "Y")
    _check(lib().sla_spmm_t(A.handle, px, py, k, _stream(stream)))
    return Y


def sla_pcg_workspace_size_multi(A: Mat, k: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().sla_pcg_workspace_size_multi(A.handle, int(k), ctypes.byref(b)))
    return b.value


def workspace_multi(A: Mat, k: int, device=None) -> torch.Tensor:
    return torch.empty(max(sla_pcg_workspace_size_multi(A, k), 1), dtype=torch.uint8,
                       device=device or A.device)


def _multi_out(st, infos, cst, k):
    return [_info(int(cst[c]), infos[c]) for c in range(k)]


def sla_pcg_solve_multi(A: Mat, G: Mat, eps: float, B: torch.Tensor,
                        X: Optional[torch.Tensor] = None, rtol: float = 1e-10, maxit: int = 1000,
                        work: Optional[torch.Tensor] = None, stream=None,
                        raise_on_error: bool = True):
    """Solve A X = B for the k columns of B (n, k) together; returns X and one
    Info per column (its own status, iterations and residual)."""
    _pair(A, G)
    k = _cols(B, A)
    pb = _block(B, A, k, "B")
    if X is None:
        X = torch.empty_like(B)
    px = _block(X, A, k, "X")
    if work is None:
        work = workspace_multi(A, k, B.device)
    pw, nw = _work(work, A)
    infos = (SolveInfo * k)()
    cst = (ctypes.c_int * k)()
    st = lib().sla_pcg_solve_multi(A.handle, G.handle, float(eps), pb, px, k, float(rtol),
                                   int(maxit), pw, nw, _stream(stream), infos, cst)
    if raise_on_error:
        _check(st, allow=(OK, NOT_CONVERGED))
    return X, _multi_out(st, infos, cst, k)


def sla_pcg_adjoint_multi(A: Mat, G: Mat, eps: float, X: torch.Tensor, GX: torch.Tensor,
                          rtol: float = 1e-10, maxit: int = 1000,
                          GB: Optional[torch.Tensor] = None,
                          grad_vals: Optional[torch.Tensor] = None,
                          work: Optional[torch.Tensor] = None, stream=None,
                          raise_on_error: bool = True):
    """Adjoint of k solves sharing A: dL/dB = A^-T dL/dX column by column and
    dL/dA on A's pattern summed over the solves."""
    _pair(A, G)
    k = _cols(X, A)
    px = _block(X, A, k, "X")
    pgx = _block(GX, A, k, "GX")
    if GB is None:
        GB = torch.empty_like(X)
    pgb = _block(GB, A, k, "GB")
    if grad_vals is None:
        grad_vals = torch.empty(A.nnz, dtype=A.dtype, device=X.device)
    pgv = _vec(grad_vals, A, A.nnz, "grad_vals")
    if work is None:
        work = workspace_multi(A, k, X.device)
    pw, nw = _work(work, A)
    infos = (SolveInfo * k)()
    cst = (ctypes.c_int * k)()
    st = lib().sla_pcg_adjoint_multi(A.handle, G.handle, float(eps), px, pgx, pgb, pgv, k,
                                     float(rtol), int(maxit), pw, nw, _stream(stream), infos, cst)
    if raise_on_error:
        _check(st, allow=(OK, NOT_CONVERGED))
    return GB, grad_vals, _multi_out(st, infos, cst, k)


def sla_pattern_grad(A: Mat, lam: torch.Tensor, x: torch.Tensor,
                     out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    pl = _vec(lam, A, A.n, "lam")
    px = _vec(x, A, A.n, "x")
    if out is None:
        out = torch.empty(A.nnz, dtype=A.dtype, device=x.device)
    po = _vec(out, A, A.nnz, "out")
    _check(lib().sla_pattern_grad(A.handle, pl, px, po, _stream(stream)))
    return out


def sla_set_profiling(enable) -> None:
    """enable: True (all classes), False, or a bit mask / iterable of class names."""
    if enable is True:
        mask = 15
    elif enable is False or enable is None:
        mask = 0
    elif isinstance(enable, int):
        mask = enable
    else:
        mask = 0
        for c in enable:
            mask |= 1 << (PROFILE_CLASSES[c] if isinstance(c, str) else int(c))
    _check(lib().sla_set_profiling(int(mask)))


def sla_set_profiling_stride(every: int) -> None:
    """Time only the launches of iterations k with k % every == 0."""
    _check(lib().sla_set_profiling_stride(int(every)))


def sla_reset_profile() -> None:
    _check(lib().sla_reset_profile())


def sla_get_profile(kernel_class) -> Tuple[int, float]:
    if isinstance(kernel_class, str):
        kernel_class = PROFILE_CLASSES[kernel_class]
    n, ms = ctypes.c_int64(), ctypes.c_double()
    _check(lib().sla_get_profile(int(kernel_class), ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def sla_status_string(status: int) -> str:
    return lib().sla_status_string(int(status)).decode()
