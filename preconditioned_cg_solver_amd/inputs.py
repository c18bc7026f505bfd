"""Seeded synthetic inputs for the PCG + factorised-SPAI solver.

This module only *builds* problem data: sparse matrices A (CSR or 3x3 BSR),
the factor G of the preconditioner, right-hand sides and loss weights.  It
performs none of the solver's arithmetic (no SpMV, no preconditioner apply, no
conjugate-gradient step, no gradient), so both sides of every parity test --
the CPU oracle and the HIP library -- can be fed from it without sharing any
of the method's code.

Workloads (the pages measure on FEM datasets that are not available; these
synthetic systems stand in for them with the same structure):

* ``poisson2d``  -- 2D 5-point Laplacian (4 on the diagonal, -1 off), Dirichlet,
  N x N interior grid.
* ``heat2d``     -- implicit-Euler heat operator I + (dt/h^2) L5 on an N x N
  interior grid, h = 1/(N+1).
* ``poisson3d``  -- 3D 7-point Laplacian (6 / -1), Dirichlet, N^3 interior grid.
* ``elastic_bsr``-- 3 dof per node, 27-point node stencil stored as 3x3 blocks,
  off-diagonal blocks -c (I + 0.1 R R^T), diagonal blocks diagonal and strictly
  dominant by 1e-2.
* ``powerlaw``   -- random SPD graph Laplacian + 1e-4 I with 16 weighted random
  neighbours per row and Zipf(2.1) column weights.

The preconditioner factor G (Learning Sparse Approximate Inverse
Preconditioners for CG on GPUs, "Approach": M^-1 = G G^T + eps I with G
sharing A's sparsity) takes the lower triangle of A's pattern (diagonal
included).  Its values are g_ii = a_ii^(-1/2) and g_ij = U(-0.1, 0.1) *
a_ii^(-1/2), the scale of every entry in row i taken from that row's diagonal.

Randomness: ``numpy.random.default_rng([config, stream, seed])`` with streams
0 = matrix values/pattern, 1 = G, 2 = right-hand side b, 3 = loss weights w,
4 = SpMV test vectors.  Draws are taken in CSR storage order of the entries
they fill.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

STREAM_MATRIX, STREAM_G, STREAM_B, STREAM_W, STREAM_X = 0, 1, 2, 3, 4


def rng_for(config: int, stream: int, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(config), int(stream), int(seed)])


@dataclasses.dataclass
class SparseMatrix:
    """Square sparse matrix in CSR (block_dim == 1) or BSR (block_dim > 1).

    ``row_ptr`` has n_block_rows + 1 int32 entries, ``col_idx`` has nnzb int32
    block-column indices sorted ascending within each row, ``vals`` has
    nnzb * block_dim**2 values, each block stored row-major.
    """

    n_block_rows: int
    block_dim: int
    row_ptr: np.ndarray
    col_idx: np.ndarray
    vals: np.ndarray

    @property
    def n(self) -> int:
        return self.n_block_rows * self.block_dim

    @property
    def nnzb(self) -> int:
        return int(self.col_idx.shape[0])

    @property
    def nnz(self) -> int:
        """Stored scalar entries."""
        return self.nnzb * self.block_dim * self.block_dim

    def astype(self, dtype) -> "SparseMatrix":
        return SparseMatrix(self.n_block_rows, self.block_dim, self.row_ptr,
                            self.col_idx, self.vals.astype(dtype))

    def row_of_entry(self) -> np.ndarray:
        """Block-row index of every stored block (int64), in storage order."""
        return np.repeat(np.arange(self.n_block_rows, dtype=np.int64),
                         np.diff(self.row_ptr.astype(np.int64)))

    def to_dense(self) -> np.ndarray:
        """Dense copy; for small matrices in tests only."""
        b = self.block_dim
        d = np.zeros((self.n, self.n), dtype=np.float64)
        rows = self.row_of_entry()
        blocks = self.vals.reshape(-1, b, b)
        for k in range(self.nnzb):
            i, j = rows[k], self.col_idx[k]
            d[i * b:(i + 1) * b, j * b:(j + 1) * b] += blocks[k]
        return d

    def to_scipy(self):
        import scipy.sparse as sp
        if self.block_dim == 1:
            return sp.csr_matrix((self.vals.astype(np.float64), self.col_idx, self.row_ptr),
                                 shape=(self.n, self.n))
        b = self.block_dim
        return sp.bsr_matrix((self.vals.reshape(-1, b, b).astype(np.float64), self.col_idx,
                              self.row_ptr), shape=(self.n, self.n)).tocsr()


# ----------------------------------------------------------------------------
# Structured stencils
# ----------------------------------------------------------------------------

def _stencil_pattern(shape, offsets):
    """CSR pattern of a stencil on a Dirichlet grid (row-major, last axis fastest).

    ``offsets`` are integer offset vectors; entries outside the grid are
    dropped.  Returns (row_ptr, col_idx, which) where ``which[k]`` is the index
    into ``offsets`` of stored entry k.  Columns come out ascending in each row
    because the offsets are visited in ascending linear-offset order.
    """
    shape = np.asarray(shape, dtype=np.int64)
    d = len(shape)
    n = int(np.prod(shape))
    strides = np.ones(d, dtype=np.int64)
    for a in range(d - 2, -1, -1):
        strides[a] = strides[a + 1] * shape[a + 1]
    offsets = [np.asarray(o, dtype=np.int64) for o in offsets]
    lin = np.array([int((o * strides).sum()) for o in offsets], dtype=np.int64)
    order = np.argsort(lin, kind="stable")
    coords = np.indices(tuple(int(s) for s in shape)).reshape(d, -1)
    rowid = np.arange(n, dtype=np.int64)
    cols = np.empty((n, len(offsets)), dtype=np.int64)
    valid = np.empty((n, len(offsets)), dtype=bool)
    for slot, oi in enumerate(order):
        c = coords + offsets[oi][:, None]
        valid[:, slot] = np.all((c >= 0) & (c < shape[:, None]), axis=0)
        cols[:, slot] = rowid + lin[oi]
    counts = valid.sum(axis=1)
    row_ptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col_idx = cols[valid]
    which = np.broadcast_to(order[None, :], cols.shape)[valid]
    return row_ptr.astype(np.int32), col_idx.astype(np.int32), which


def _laplacian(shape, diag: float, off: float) -> SparseMatrix:
    d = len(shape)
    offs = [np.zeros(d, dtype=np.int64)]
    for a in range(d):
        for s in (-1, 1):
            o = np.zeros(d, dtype=np.int64)
            o[a] = s
            offs.append(o)
    rp, ci, which = _stencil_pattern(shape, offs)
    vals = np.where(which == 0, diag, off).astype(np.float64)
    return SparseMatrix(int(np.prod(shape)), 1, rp, ci, vals)


def poisson2d(N: int) -> SparseMatrix:
    """5-point Laplacian on an N x N interior grid: 4 on the diagonal, -1 off."""
    return _laplacian((N, N), 4.0, -1.0)


def poisson3d(N: int) -> SparseMatrix:
    """7-point Laplacian on an N^3 interior grid: 6 on the diagonal, -1 off."""
    return _laplacian((N, N, N), 6.0, -1.0)


def heat_scale(N: int, dt: float = 1e-2) -> float:
    """dt / h^2 with h = 1/(N+1)."""
    return dt * float(N + 1) ** 2


def heat2d(N: int, dt: float = 1e-2) -> SparseMatrix:
    """Implicit-Euler heat operator I + (dt/h^2) L5 on an N x N interior grid."""
    s = heat_scale(N, dt)
    return _laplacian((N, N), 1.0 + 4.0 * s, -s)


# ----------------------------------------------------------------------------
# Elasticity-like 3x3 block system
# ----------------------------------------------------------------------------

def elastic_bsr(N: int, rng: np.random.Generator, margin: float = 1e-2) -> SparseMatrix:
    """3 dof per node on an N^3 node grid, 27-point node stencil, 3x3 BSR.

    Off-diagonal block pairs I < J draw c ~ U(0.5, 1) and R ~ N(0,1)^{3x3};
    block(I,J) = block(J,I) = -c (I3 + 0.1 R R^T).  Diagonal blocks are
    diagonal with a_ii = sum_j |a_ij| (j != i) + margin, which makes A strictly
    diagonally dominant with a positive diagonal, hence SPD.
    """
    offs = [np.array([a, b, c], dtype=np.int64)
            for a in (-1, 0, 1) for b in (-1, 0, 1) for c in (-1, 0, 1)]
    rp, ci, _ = _stencil_pattern((N, N, N), offs)
    nb = N ** 3
    nnzb = ci.shape[0]
    rows = np.repeat(np.arange(nb, dtype=np.int64), np.diff(rp.astype(np.int64)))
    cols = ci.astype(np.int64)
    upper = cols > rows
    up_keys = rows[upper] * nb + cols[upper]          # ascending (CSR order)
    npairs = up_keys.shape[0]
    c = rng.uniform(0.5, 1.0, size=npairs)
    R = rng.standard_normal(size=(npairs, 3, 3))
    B = -c[:, None, None] * (np.eye(3)[None] + 0.1 * np.einsum("pij,pkj->pik", R, R))
    B = 0.5 * (B + np.transpose(B, (0, 2, 1)))         # exact symmetry
    pair = np.full(nnzb, -1, dtype=np.int64)
    pair[upper] = np.arange(npairs)
    lower = cols < rows
    pair[lower] = np.searchsorted(up_keys, cols[lower] * nb + rows[lower])
    vals = np.zeros((nnzb, 3, 3), dtype=np.float64)
    offd = pair >= 0
    vals[offd] = B[pair[offd]]
    # diagonal of each scalar row
    absrow = np.abs(vals[offd]).sum(axis=2)           # (noff, 3)
    rowsum = np.zeros((nb, 3), dtype=np.float64)
    np.add.at(rowsum, rows[offd], absrow)
    diag = rowsum + margin
    dpos = np.nonzero(cols == rows)[0]
    vals[dpos, 0, 0] = diag[:, 0]
    vals[dpos, 1, 1] = diag[:, 1]
    vals[dpos, 2, 2] = diag[:, 2]
    return SparseMatrix(nb, 3, rp, ci, vals.reshape(-1))


# ----------------------------------------------------------------------------
# Power-law random SPD
# ----------------------------------------------------------------------------

def powerlaw_spd(n: int, rng: np.random.Generator, k: int = 16, exponent: float = 2.1,
                 shift: float = 1e-4) -> SparseMatrix:
    """Weighted random graph Laplacian + shift*I with power-law column degrees.

    Column weights w_j ~ Zipf(exponent) (capped at n); every row picks k
    distinct columns j != i with probability proportional to w_j; the picked
    entries get -U(0,1); A_off = B + B^T (duplicates summed) and
    a_ii = sum_{j != i} |a_ij| + shift.
    """
    import scipy.sparse as sp
    w = np.minimum(rng.zipf(exponent, size=n), n).astype(np.float64)
    cw = np.cumsum(w)
    total = cw[-1]
    picks = np.zeros((n, k), dtype=np.int64)
    need = np.ones((n, k), dtype=bool)
    rows_all = np.arange(n, dtype=np.int64)
    active = rows_all
    while active.size:
        sub = picks[active]
        ridx, sidx = np.nonzero(need[active])
        u = rng.uniform(0.0, total, size=ridx.shape[0])
        sub[ridx, sidx] = np.minimum(np.searchsorted(cw, u, side="right"), n - 1)
        # reject self loops and repeats within a row (keep the first occurrence)
        order = np.argsort(sub, axis=1, kind="stable")
        srt = np.take_along_axis(sub, order, axis=1)
        dup_sorted = np.zeros(sub.shape, dtype=bool)
        dup_sorted[:, 1:] = srt[:, 1:] == srt[:, :-1]
        dup = np.zeros(sub.shape, dtype=bool)
        np.put_along_axis(dup, order, dup_sorted, axis=1)
        subneed = dup | (sub == active[:, None])
        picks[active] = sub
        need[active] = subneed
        active = active[subneed.any(axis=1)]
    bvals = -rng.uniform(0.0, 1.0, size=(n, k))
    r = np.repeat(rows_all, k)
    c = picks.reshape(-1)
    v = bvals.reshape(-1)
    Boff = sp.coo_matrix((v, (r, c)), shape=(n, n)).tocsr()
    Aoff = (Boff + Boff.T).tocsr()
    Aoff.sum_duplicates()
    Aoff.sort_indices()
    diag = np.asarray(np.abs(Aoff).sum(axis=1)).reshape(-1) + shift
    A = (Aoff + sp.diags(diag)).tocsr()
    A.sum_duplicates()
    A.sort_indices()
    return SparseMatrix(n, 1, A.indptr.astype(np.int32), A.indices.astype(np.int32),
                        A.data.astype(np.float64))


# ----------------------------------------------------------------------------
# Preconditioner factor G on the lower-triangular pattern of A
# ----------------------------------------------------------------------------

def spai_factor(A: SparseMatrix, rng: np.random.Generator, spread: float = 0.1) -> SparseMatrix:
    """G on tril(A) (block-lower for BSR, diagonal block kept whole).

    Scalar entry (i, j) of G: a_ii^(-1/2) on the diagonal, U(-spread, spread) *
    a_ii^(-1/2) elsewhere, one draw per off-diagonal stored scalar in storage
    order.
    """
    b = A.block_dim
    rows = A.row_of_entry()
    cols = A.col_idx.astype(np.int64)
    keep = cols <= rows
    counts = np.bincount(rows[keep], minlength=A.n_block_rows)
    rp = np.zeros(A.n_block_rows + 1, dtype=np.int64)
    np.cumsum(counts, out=rp[1:])
    gcols = cols[keep]
    grows = rows[keep]
    nnzb = gcols.shape[0]
    # scalar diagonal of A
    blocks = A.vals.reshape(-1, b, b)
    dpos = np.nonzero(cols == rows)[0]
    if dpos.shape[0] != A.n_block_rows:
        raise ValueError("every row of A must store its diagonal")
    adiag = np.empty(A.n, dtype=np.float64)
    for r in range(b):
        adiag[rows[dpos] * b + r] = blocks[dpos, r, r]
    if np.any(adiag <= 0):
        raise ValueError("A must have a positive diagonal")
    scale = 1.0 / np.sqrt(adiag)                         # a_ii^(-1/2)
    g = np.empty((nnzb, b, b), dtype=np.float64)
    is_diag_scalar = np.zeros((nnzb, b, b), dtype=bool)
    on_diag_block = gcols == grows
    for r in range(b):
        is_diag_scalar[on_diag_block, r, r] = True
    n_off = int((~is_diag_scalar).sum())
    u = rng.uniform(-spread, spread, size=n_off)
    srow = (grows[:, None, None] * b + np.arange(b)[None, :, None]) * np.ones((1, 1, b), np.int64)
    sc = scale[srow]
    g[is_diag_scalar] = sc[is_diag_scalar]
    g[~is_diag_scalar] = u * sc[~is_diag_scalar]
    return SparseMatrix(A.n_block_rows, b, rp.astype(np.int32), gcols.astype(np.int32),
                        g.reshape(-1))


def diagonal_factor(A: SparseMatrix) -> SparseMatrix:
    """G = diag(a_ii^(-1/2)) in A's format (3x3 diagonal blocks for BSR); with
    eps = 0, M^-1 = G G^T is Jacobi (diagonal) preconditioning."""
    b = A.block_dim
    rows = A.row_of_entry()
    dpos = np.nonzero(A.col_idx.astype(np.int64) == rows)[0]
    if dpos.shape[0] != A.n_block_rows:
        raise ValueError("every row of A must store its diagonal")
    blocks = A.vals.reshape(-1, b, b)
    d = np.stack([blocks[dpos, r, r] for r in range(b)], axis=1)      # (nbr, b)
    g = np.zeros((A.n_block_rows, b, b), dtype=np.float64)
    for r in range(b):
        g[:, r, r] = 1.0 / np.sqrt(d[:, r])
    rp = np.arange(A.n_block_rows + 1, dtype=np.int32)
    return SparseMatrix(A.n_block_rows, b, rp, np.arange(A.n_block_rows, dtype=np.int32),
                        g.reshape(-1))


# ----------------------------------------------------------------------------
# Right-hand sides
# ----------------------------------------------------------------------------

def smooth_field_2d(N: int, rng: np.random.Generator, modes: int = 8) -> np.ndarray:
    """Sum of `modes` random separable sinusoids on the N x N interior grid
    (x = i h, h = 1/(N+1)), min-max rescaled to [0, 1]."""
    h = 1.0 / (N + 1)
    a = rng.uniform(0.0, 1.0, size=modes)
    kk = rng.integers(1, 9, size=modes)
    ll = rng.integers(1, 9, size=modes)
    ph = rng.uniform(0.0, 2 * math.pi, size=modes)
    ps = rng.uniform(0.0, 2 * math.pi, size=modes)
    y = (np.arange(N) + 1) * h
    x = (np.arange(N) + 1) * h
    f = np.zeros((N, N), dtype=np.float64)
    for m in range(modes):
        f += a[m] * np.outer(np.sin(math.pi * ll[m] * y + ps[m]),
                             np.sin(math.pi * kk[m] * x + ph[m]))
    lo, hi = f.min(), f.max()
    f = (f - lo) / (hi - lo) if hi > lo else np.zeros_like(f)
    return f.reshape(-1)


# ----------------------------------------------------------------------------
# The five workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Problem:
    name: str
    config: int
    A: SparseMatrix
    G: SparseMatrix
    b: np.ndarray
    eps: float
    rtol: float
    maxit: int
    loss: str                       # "sumsq" (L = sum x^2) or "dot" (L = <w, x>)
    w: Optional[np.ndarray] = None
    dtype: str = "f64"

    def astype(self, dtype: str) -> "Problem":
        npdt = np.float32 if dtype == "f32" else np.float64
        return dataclasses.replace(
            self, A=self.A.astype(npdt), G=self.G.astype(npdt), b=self.b.astype(npdt),
            w=None if self.w is None else self.w.astype(npdt), dtype=dtype)


CONFIG_NAMES = {0: "poisson2d_32", 1: "heat2d_512", 2: "poisson3d_128",
                3: "elastic_bsr3_64", 4: "powerlaw_4M"}
DEFAULT_SIZE = {0: 32, 1: 512, 2: 128, 3: 64, 4: 4_194_304}


def make_problem(config: int, dtype: str = "f64", seed: int = 0,
                 size: Optional[int] = None) -> Problem:
    """Build workload `config` (0..4).  `size` overrides the grid edge (0-3)
    or the row count (4) for scaled-down tests."""
    N = DEFAULT_SIZE[config] if size is None else int(size)
    rm, rg, rb, rw = (rng_for(config, s, seed) for s in (STREAM_MATRIX, STREAM_G, STREAM_B, STREAM_W))
    w = None
    if config == 0:
        A = poisson2d(N)
        b = rb.uniform(-1.0, 1.0, size=A.n)
        eps, rtol, maxit, loss = 3e-3, 1e-10, 2000, "sumsq"
    elif config == 1:
        A = heat2d(N)
        b = smooth_field_2d(N, rb)
        eps, rtol, maxit, loss = 3e-3, 1e-8, 5000, "sumsq"
    elif config == 2:
        A = poisson3d(N)
        b = rb.standard_normal(A.n)
        w = rw.standard_normal(A.n)
        eps, rtol, maxit, loss = 3e-3, 1e-10, 5000, "dot"
    elif config == 3:
        A = elastic_bsr(N, rm)
        b = rb.standard_normal(A.n)
        w = rw.standard_normal(A.n)
        eps, rtol, maxit, loss = 3e-3, 1e-8, 5000, "dot"
    elif config == 4:
        A = powerlaw_spd(N, rm)
        b = rb.standard_normal(A.n)
        w = rw.standard_normal(A.n)
        eps, rtol, maxit, loss = 3e-3, 1e-8, 5000, "dot"
    else:
        raise ValueError(f"unknown config {config}")
    G = spai_factor(A, rg)
    p = Problem(CONFIG_NAMES[config] if size is None else f"{CONFIG_NAMES[config]}@{N}",
                config, A, G, b.astype(np.float64), eps, rtol, maxit, loss, w)
    return p.astype(dtype) if dtype != "f64" else p


def loss_grad_weights(p: Problem, x: np.ndarray) -> np.ndarray:
    """dL/dx for the problem's loss: 2x for L = sum x^2, w for L = <w, x>.
    (Input preparation for the adjoint solve, given x.)"""
    if p.loss == "sumsq":
        return 2.0 * x
    return p.w


def spmv_test_vector(config: int, n: int, seed: int = 0, dtype=np.float64) -> np.ndarray:
    return rng_for(config, STREAM_X, seed).standard_normal(n).astype(dtype)


def random_spd_csr(n: int, rng: np.random.Generator, min_deg: int = 0, max_deg: int = 12,
                   margin: float = 1e-2, long_rows: int = 0, long_deg: int = 0) -> SparseMatrix:
    """Irregular symmetric, strictly diagonally dominant CSR matrix for edge
    cases: rows get U{min_deg..max_deg} random neighbours, `long_rows` rows
    get `long_deg` neighbours (capped at n-1)."""
    import scipy.sparse as sp
    deg = rng.integers(min_deg, max_deg + 1, size=n)
    if long_rows:
        hubs = rng.choice(n, size=min(long_rows, n), replace=False)
        deg[hubs] = min(long_deg, n - 1)
    r = np.repeat(np.arange(n, dtype=np.int64), deg)
    c = np.concatenate([rng.choice(n, size=d, replace=False) if d else np.empty(0, np.int64)
                        for d in deg]).astype(np.int64) if n else np.empty(0, np.int64)
    keep = r != c
    r, c = r[keep], c[keep]
    v = -rng.uniform(0.1, 1.0, size=r.shape[0])
    B = sp.coo_matrix((v, (r, c)), shape=(n, n)).tocsr()
    Aoff = (B + B.T).tocsr()
    Aoff.sum_duplicates()
    diag = np.asarray(np.abs(Aoff).sum(axis=1)).reshape(-1) + margin
    A = (Aoff + sp.diags(diag)).tocsr()
    A.sum_duplicates()
    A.sort_indices()
    return SparseMatrix(n, 1, A.indptr.astype(np.int32), A.indices.astype(np.int32),
                        A.data.astype(np.float64))
