/*
 * sla.h -- C ABI of the MI355X (gfx950) preconditioned conjugate-gradient
 * library: CG for sparse symmetric positive-definite A x = b, preconditioned
 * by the factorised sparse approximate inverse M^-1 = G G^T + eps I, and the
 * adjoint (backward) solve of that system.
 *
 * Method (pages cited by title and section):
 *  - "Learning Sparse Approximate Inverse Preconditioners for Conjugate
 *    Gradient Solvers on GPUs", "Approach": M^-1 = G G^T + eps I with G on
 *    A's sparsity, so a preconditioner apply is two sparse products; "Problem":
 *    CG for sparse SPD systems on GPUs.  G here has the lower-triangular
 *    (block-lower) part of A's pattern.
 *  - "torch-sla: Differentiable Sparse Linear Algebra with Adjoint Solvers...",
 *    Technical Summary, Methodology 2 (adjoint differentiation, linear
 *    systems): the backward pass is one solve A^T lambda = dL/dx, and
 *    dL/dA_ij = -lambda_i x_j on the sparsity pattern only; memory is
 *    O(n + nnz) and independent of the iteration count.
 *
 * Conventions shared by every entry point:
 *  - All array arguments named d_* are DEVICE pointers (memory of the current
 *    HIP device, e.g. from hipMalloc or a torch CUDA tensor).  Index arrays
 *    are int32; value arrays are fp64 (SLA_F64) or fp32 (SLA_F32) as given at
 *    create time.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    device work is enqueued on it.  sla_spmv returns without waiting;
 *    sla_csr_create / sla_bsr_create, sla_pcg_solve and sla_pcg_adjoint
 *    return after their results are final (they synchronise `stream`).
 *  - Errors are returned as sla_status, never thrown; sla_last_error() gives
 *    a thread-local message for the last failing call on that thread.
 *  - Nothing here falls back to the CPU: every numerical step runs in the
 *    library's HIP kernels.
 *  - Device memory that a handle owns (explicit transpose, sliced copies,
 *    tiles, scratch) comes from a caching allocator in the library:
 *    sla_mat_destroy parks the buffers in a per-device cache (up to 8 GiB;
 *    beyond that they are freed) and later handles reuse them, so
 *    re-creating handles every step costs no hipMalloc / hipFree.  A failed
 *    allocation empties the cache and retries.  Cached buffers are held
 *    until the process ends.
 *
 * Environment variables (all optional; the defaults are the measured best
 * choices and no result depends on them beyond rounding order):
 *  - SLA_FUSION=fused|unfused: iteration form of the one-right-hand-side
 *    solves (default: fused for CSR matrices in the sliced layout, separate
 *    streaming passes otherwise).  SLA_MFUSION=fused: the same for the
 *    multi-right-hand-side solves (default: separate).
 *  - SLA_MCHUNK=1|2|4|8: most columns a multi-right-hand-side pass takes
 *    (default: 8, or 4 for a sliced CSR matrix reaching far from its
 *    diagonal).
 *  - SLA_SMALL=0: no one-workgroup solve for systems of at most 1024 rows.
 *  - SLA_SELL=0: no sliced (SELL-64 / BSR sliced-ELL) copies at create time;
 *    SLA_SELL16=0: absolute int32 columns in them instead of 16-bit offsets;
 *    SLA_SELL_OFS=0: no slice-offset form (by default a CSR matrix whose
 *    64-row slices each have at most 8 distinct column offsets over sorted
 *    rows, as stencils do, stores one offset per slot of a slice and a
 *    one-byte mask of present slots per row, and its products, for one or
 *    several right-hand sides, read no per-entry column words).
 *  - SLA_GRID=G (G >= 8, rounded down to a multiple of 8): workgroups of the
 *    row-parallel kernels instead of the resident capacity.
 *  - SLA_MALL_BUDGET_MB (default 208) and SLA_MALL_POLICY=A|G|AG|AT|all|none:
 *    which operators a solve keeps resident in the 256 MB Infinity Cache
 *    (G = G and G^T, AG = A and G, AT = A and G^T).  Default: all three when
 *    they fit the budget with eight vectors; else G and G^T when the bytes
 *    their products stream are at least A's and fit 240 MB beside six
 *    vectors; else A when it fits the budget; else none.  The rest stream
 *    non-temporally.
 *  - SLA_BATCH_ITERS (1..4096): the full batch of iterations enqueued
 *    between two host polls of the device's record (default: sized from an
 *    estimate of one iteration to last about 0.8 ms, 2..16; the last
 *    batches of a solve are shortened to the predicted stopping iteration).
 *  - SLA_ORDER=0|1: locality ordering of the solves off, or on for every CSR
 *    matrix outside the SELL layout (default: automatic, see
 *    sla_mat_reordered).
 *  - SLA_COLBLK=0: the separate iteration form on a locality ordering keeps
 *    the row tiles instead of splitting each operator into 8 column blocks
 *    (read at handle creation).
 *  - SLA_WIN=0|1|2: the windowed slice-offset engine off, for the A steps
 *    (default), or for every step.
 *  - SLA_TRACE=1: roctx ranges around handle creation, the locality
 *    ordering, solves, adjoint solves and the pattern gradient (seen by
 *    rocprofv3 --marker-trace; the roctx library is opened at run time),
 *    and one line per call on stderr with n, iterations, relative residual,
 *    status and wall time.
 * SLA_GRID is read once per device, SLA_MALL_BUDGET_MB, SLA_BATCH_ITERS,
 * SLA_MCHUNK and SLA_TRACE once per process; the others at every handle
 * creation or solve.
 */
#ifndef SLA_H
#define SLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* SLA_DTYPE_RANGE_ makes every non-negative int32 a value of the type, so a
 * caller's out-of-range dtype reaches the library's check (and is rejected
 * with SLA_ERR_INVALID_ARG) instead of being an invalid enum value. */
typedef enum { SLA_F64 = 0, SLA_F32 = 1, SLA_DTYPE_RANGE_ = 0x7fffffff } sla_dtype;

typedef enum {
    SLA_OK = 0,
    SLA_NOT_CONVERGED = 1,       /* > 0: result valid (last iterate), warning   */
    SLA_ERR_INVALID_ARG = -1,    /* bad size, pointer, dtype, CSR structure     */
    SLA_ERR_UNSUPPORTED = -2,    /* e.g. block size other than 1 or 3, n>=2^31  */
    SLA_ERR_BREAKDOWN = -3,      /* p.Ap <= 0, r.z <= 0 or non-finite residual  */
    SLA_ERR_NONFINITE = -4,      /* right-hand side holds NaN/Inf               */
    SLA_ERR_HIP = -5,            /* a HIP runtime call failed                   */
    SLA_ERR_OOM = -6             /* device or pinned host allocation failed     */
} sla_status;

/* Flags for sla_csr_create / sla_bsr_create. */
#define SLA_BUILD_TRANSPOSE 1u   /* build and keep the explicit transpose (needed for G) */
#define SLA_VALIDATE 2u          /* check the structure on the device (O(nnz))          */

typedef struct sla_mat *sla_mat_t;

typedef struct {
    int32_t iterations;   /* number of products with A (= x updates) performed  */
    int32_t converged;    /* 1 if ||r_k|| <= rtol ||b|| was reached               */
    double rel_residual;  /* ||r_k|| / ||b|| of the recursive residual (0 if b=0) */
    double bnorm;         /* ||b||_2 of the right-hand side actually solved       */
} sla_solve_info;

/*
 * Create a handle for a square CSR matrix with n rows and nnz stored entries.
 * The handle BORROWS d_row_ptr[n+1], d_col_idx[nnz] (columns ascending within
 * each row, no duplicates, 0 <= col < n) and d_vals[nnz]; they must stay alive
 * and unchanged until sla_mat_destroy.  The handle OWNS what it derives at
 * create time: the SpMV tiling of the rows (row binning by nonzeros per row)
 * and, with SLA_BUILD_TRANSPOSE, an explicit transpose in CSR built once on
 * the device (a stable sort of the entries by column, so every transposed row
 * lists its columns ascending and later products need no atomics).
 * Errors: SLA_ERR_INVALID_ARG (negative sizes, NULL pointers with nnz > 0,
 * row_ptr[n] != nnz, or -- with SLA_VALIDATE -- a malformed structure),
 * SLA_ERR_UNSUPPORTED (n or nnz >= 2^31), SLA_ERR_OOM, SLA_ERR_HIP.
 */
sla_status sla_csr_create(sla_mat_t *out, int64_t n, int64_t nnz, const int32_t *d_row_ptr,
                          const int32_t *d_col_idx, const void *d_vals, sla_dtype dtype,
                          uint32_t flags, void *stream);

/*
 * Same for a square block-sparse matrix of n_block_rows x n_block_rows blocks
 * of size block_dim x block_dim (only block_dim 3 and 1 are supported):
 * d_brow_ptr[n_block_rows+1], d_bcol_idx[nnzb], d_bvals[nnzb*block_dim^2]
 * with every block stored row-major.  The transpose (SLA_BUILD_TRANSPOSE)
 * transposes the block pattern and every block.
 */
sla_status sla_bsr_create(sla_mat_t *out, int64_t n_block_rows, int64_t nnzb, int32_t block_dim,
                          const int32_t *d_brow_ptr, const int32_t *d_bcol_idx,
                          const void *d_bvals, sla_dtype dtype, uint32_t flags, void *stream);

/* Release the handle and everything it owns (the borrowed arrays are
 * untouched).  Waits for the asynchronous calls queued on the handle (the
 * products, preconditioner apply, pattern gradient and SAI loss record an
 * event on their stream), not for the rest of the device, so it may be
 * called right after them; the handle's buffers then go to the library's
 * buffer cache.  Handles may be used from several streams and threads at
 * once, except that the first solve with a reordered A (sla_mat_reordered)
 * builds the permuted copies and must not overlap other calls on the same
 * handles. */
sla_status sla_mat_destroy(sla_mat_t m);

/* Sizes of a handle: scalar rows, stored scalar entries, block size, dtype. */
sla_status sla_mat_info(sla_mat_t m, int64_t *n, int64_t *nnz, int32_t *block_dim,
                        int32_t *dtype);

/*
 * Device arrays of the explicit transpose owned by the handle (built with
 * SLA_BUILD_TRANSPOSE): row_ptr[n_block_rows+1], col_idx[nnzb], vals.  The
 * pointers stay valid until sla_mat_destroy; the caller must not free them.
 * Error: SLA_ERR_INVALID_ARG if the handle has no transpose.
 */
sla_status sla_mat_transpose_arrays(sla_mat_t m, const int32_t **d_row_ptr,
                                    const int32_t **d_col_idx, const void **d_vals);

/* Number of SpMV tiles (row bins) of the handle and how many of them are long
 * rows processed by row splitting; for tests and reports. */
sla_status sla_mat_tiling(sla_mat_t m, int32_t transpose, int64_t *n_tiles, int64_t *n_long);

/*
 * Whether the solves (sla_pcg_solve, sla_pcg_solve_history, sla_pcg_adjoint
 * and their several-right-hand-side forms) with m as A run on a locality
 * ordering: *reordered = 1 or
 * 0, decided when m was created.  Such a solve applies one symmetric
 * permutation P to the whole system (P A P^T y = P b with the preconditioner
 * P G G^T P^T + eps I, which is P M^-1 P^T, so the iterates are those of the
 * unpermuted solve up to rounding order) and returns x = P^T y; dL/dA is
 * still computed on A's own storage order.  P sorts the rows by decreasing
 * length, so the most-referenced entries of the gathered vectors share cache
 * lines, and deals them round-robin over eight contiguous row segments, so
 * the per-XCD shares of the row-parallel kernels get the same mix of long
 * and short rows.  It applies to CSR matrices outside the SELL layout with
 * at least 131072 rows whose sampled stored entries lie mostly more than
 * 32768 rows from the diagonal (random-graph-like gathers with no locality
 * to lose); SLA_ORDER=0 turns it off and SLA_ORDER=1 applies it to every
 * CSR matrix outside the SELL layout.  The first such solve builds P (on
 * the device), P A P^T into A's handle and P G P^T into G's handle (G's copy
 * is rebuilt when G is next used with another reordered A); they stay until
 * the handles are destroyed, so the handles then hold twice their matrices'
 * memory.  That first solve is synchronous set-up work and must not overlap
 * other calls on the same handles.  The workspace of such an A holds two
 * more n-vectors (sla_pcg_workspace_size includes them).  The several-
 * right-hand-side solves (sla_pcg_solve_multi, sla_pcg_adjoint_multi) use
 * the same ordering, permuting the n x k blocks by rows; their workspace
 * holds two more n x k blocks (sla_pcg_workspace_size_multi includes them).
 */
sla_status sla_mat_reordered(sla_mat_t m, int32_t *reordered);

/* y = A x (transpose = 0) or y = A^T x via the explicit transpose (transpose = 1).
 * d_x[n] and d_y[n] must not overlap.  Asynchronous on `stream`. */
sla_status sla_spmv(sla_mat_t A, const void *d_x, void *d_y, void *stream);
sla_status sla_spmv_t(sla_mat_t A, const void *d_x, void *d_y, void *stream);

/*
 * Bytes of device workspace that sla_pcg_solve / sla_pcg_adjoint /
 * sla_precond_apply need for a system of A's size: O(n) (seven vectors, the
 * per-workgroup reduction partials and a small solver state), independent of
 * maxit.  The caller allocates it (alignment 256 bytes) and passes it in; the
 * library keeps nothing in it between calls.
 */
sla_status sla_pcg_workspace_size(sla_mat_t A, size_t *bytes);

/*
 * z = (G G^T + eps I) r  (the preconditioner apply), with G^T the handle's
 * explicit transpose.  d_r[n], d_z[n] device vectors, workspace as above.
 * Asynchronous on `stream`.
 */
sla_status sla_precond_apply(sla_mat_t G, double eps, const void *d_r, void *d_z, void *d_work,
                             size_t work_bytes, void *stream);

/*
 * Preconditioned CG for A x = b, M^-1 = G G^T + eps I, x_0 = 0.
 * A: SPD (assumed, not checked); G: same size, block size and dtype as A,
 * created with SLA_BUILD_TRANSPOSE.  d_b[n] input, d_x[n] output (must not
 * alias d_b or the workspace).  Stops when the recursive residual satisfies
 * ||r_k||_2 <= rtol ||b||_2 (tested after each residual update, before the
 * preconditioner) or after maxit iterations.  Returns SLA_OK (converged,
 * including b = 0 with 0 iterations), SLA_NOT_CONVERGED (maxit reached; d_x
 * holds the last iterate), SLA_ERR_BREAKDOWN (p.Ap <= 0, r.z <= 0 or a
 * non-finite residual; d_x holds the last complete iterate),
 * SLA_ERR_NONFINITE (b holds NaN/Inf), SLA_ERR_INVALID_ARG (mismatched
 * handles, eps < 0, rtol < 0, maxit < 0, workspace too small).  `info` (may
 * be NULL) receives iterations, convergence and residual.
 */
sla_status sla_pcg_solve(sla_mat_t A, sla_mat_t G, double eps, const void *d_b, void *d_x,
                         double rtol, int32_t maxit, void *d_work, size_t work_bytes, void *stream,
                         sla_solve_info *info);

/*
 * sla_pcg_solve that also records the CG coefficients, for spectral estimates
 * of the preconditioned operator (the Lanczos tridiagonal of M^-1 A is built
 * from them: T_jj = 1/alpha_j + beta_{j-1}/alpha_{j-1}, T_j,j+1 =
 * sqrt(beta_j)/alpha_j).  d_alpha[k-1] = alpha_k (k = 1 .. iterations) and
 * d_beta[k-1] = beta_k = rho_k / rho_{k-1} (k = 1 .. iterations - 1), for
 * k <= hist_len; both are caller-owned device arrays of hist_len doubles
 * (entries past the iterations performed are left untouched).  Other
 * arguments and statuses as sla_pcg_solve; SLA_ERR_INVALID_ARG if
 * hist_len < 0 or a buffer is NULL with hist_len > 0.
 */
sla_status sla_pcg_solve_history(sla_mat_t A, sla_mat_t G, double eps, const void *d_b,
                                 void *d_x, double rtol, int32_t maxit, void *d_work,
                                 size_t work_bytes, double *d_alpha, double *d_beta,
                                 int32_t hist_len, void *stream, sla_solve_info *info);

/*
 * Adjoint of x = A^-1 b for a scalar loss L(x) with gradient d_grad_x = dL/dx:
 * solves A^T lambda = dL/dx with the same preconditioner (A^T = A for the SPD
 * matrices this solver targets), writes dL/db = lambda to d_grad_b[n], and
 * dL/dA at every stored scalar entry (i, j) = -lambda_i x_j to
 * d_grad_vals[nnz] in A's storage order (BSR: block by block, row-major).
 * d_x is the forward solution.  Statuses as for sla_pcg_solve; the gradient
 * is written whenever lambda is (SLA_OK or SLA_NOT_CONVERGED).
 */
sla_status sla_pcg_adjoint(sla_mat_t A, sla_mat_t G, double eps, const void *d_x,
                           const void *d_grad_x, void *d_grad_b, void *d_grad_vals, double rtol,
                           int32_t maxit, void *d_work, size_t work_bytes, void *stream,
                           sla_solve_info *info);

/*
 * Several right-hand sides sharing A (and G).  Multi-vectors are n x k
 * row-major device arrays in A's dtype: entry i of column c at [i * k + c],
 * so one gathered matrix column brings in the k values of that row at once.
 * Batched same-pattern solves are the batched use of "torch-sla"
 * (Significance); the k solves share only the operators.
 */

/* Y = A X (sla_spmm) or Y = A^T X (sla_spmm_t, needs SLA_BUILD_TRANSPOSE) for
 * k >= 0 columns.  Asynchronous on `stream`.  SLA_ERR_INVALID_ARG on a NULL
 * handle, k < 0, or NULL / aliased X and Y. */
sla_status sla_spmm(sla_mat_t A, const void *d_x, void *d_y, int32_t k, void *stream);
sla_status sla_spmm_t(sla_mat_t A, const void *d_x, void *d_y, int32_t k, void *stream);

/* Device workspace bytes for sla_pcg_solve_multi / sla_pcg_adjoint_multi
 * with k right-hand sides (k >= 1). */
sla_status sla_pcg_workspace_size_multi(sla_mat_t A, int32_t k, size_t *bytes);

/*
 * Solve A X = B for the k >= 1 columns of B with the preconditioner
 * M^-1 = G G^T + eps I.  Every column is its own PCG solve with the stopping
 * rule, statuses and results of sla_pcg_solve (column c of X equals the
 * one-right-hand-side solve of column c of B, to rounding); the columns are
 * advanced together, up to 8 per pass, so each product streams the matrix
 * once for all of them.  A column that exits is frozen while the others go
 * on.  info[k] and col_status[k] (host arrays, either may be NULL) receive
 * each column's record and status.  Returns the first column error if any
 * column failed (SLA_ERR_BREAKDOWN, SLA_ERR_NONFINITE), else
 * SLA_NOT_CONVERGED if any column hit maxit, else SLA_OK; X is written for
 * every column.  Synchronous with respect to the host (returns when done).
 */
sla_status sla_pcg_solve_multi(sla_mat_t A, sla_mat_t G, double eps, const void *d_b, void *d_x,
                               int32_t k, double rtol, int32_t maxit, void *d_work,
                               size_t work_bytes, void *stream, sla_solve_info *info,
                               sla_status *col_status);

/*
 * Adjoint of X = A^-1 B over k solves sharing A, for a loss with gradient
 * d_grad_x = dL/dX (n x k): d_grad_b = dL/dB solves A^T Lambda = dL/dX column
 * by column, and d_grad_vals[nnz] = dL/dA on A's pattern, summed over the
 * solves: -sum_c Lambda[i, c] X[j, c] at every stored scalar (i, j), in A's
 * storage order ("torch-sla", Technical Summary, Methodology 2, with the
 * gradients of the k uses of A added).  Statuses as sla_pcg_solve_multi; the
 * gradient is written unless a column failed.
 */
sla_status sla_pcg_adjoint_multi(sla_mat_t A, sla_mat_t G, double eps, const void *d_x,
                                 const void *d_grad_x, void *d_grad_b, void *d_grad_vals,
                                 int32_t k, double rtol, int32_t maxit, void *d_work,
                                 size_t work_bytes, void *stream, sla_solve_info *info,
                                 sla_status *col_status);

/*
 * Extreme Ritz values of M^-1 A from k steps of PCG: the smallest and largest
 * eigenvalues of the Lanczos tridiagonal built from h_alpha[0..k-1] and
 * h_beta[0..k-2] as recorded by sla_pcg_solve_history (host arrays).  They lie
 * inside [lambda_min, lambda_max] of M^-1 A and approach its ends as k grows,
 * so *lmax / *lmin estimates the preconditioned condition number, one of the
 * metrics of "Learning Sparse Approximate Inverse Preconditioners for
 * Conjugate Gradient Solvers on GPUs" (Experimental setup).  Host-only and
 * synchronous.  SLA_ERR_INVALID_ARG if k < 1, a pointer is NULL, an alpha is
 * not finite and > 0, or a beta is not finite and >= 0.
 */
sla_status sla_lanczos_extremes(const double *h_alpha, const double *h_beta, int32_t k,
                                double *lmin, double *lmax);

/*
 * Stochastic estimate of the scale-invariant SAI loss || A M^-1 / scale - I ||_F^2
 * that the learned factor is trained on (same paper, Approach), for a given G:
 * for each probe w_j, column j of the column-major n x nprobe device array
 * d_probes (A's dtype), d_out[j] = || A (G G^T w_j + eps w_j) / scale - w_j ||^2
 * (device double).  For probes with E[w w^T] = I (Rademacher or Gaussian) the
 * mean of d_out estimates the loss; with the n unit vectors as probes the sum
 * is the loss exactly.  scale is the caller's matrix norm.  G must carry its
 * transpose; d_work needs max(sla_pcg_workspace_size(A), ..(G)) bytes.
 * Asynchronous on `stream`.  SLA_ERR_INVALID_ARG on NULL or mismatched
 * handles, eps < 0, scale <= 0, nprobe < 0 or a short workspace.
 */
sla_status sla_sai_loss(sla_mat_t A, sla_mat_t G, double eps, const void *d_probes,
                        int32_t nprobe, double scale, void *d_work, size_t work_bytes,
                        double *d_out, void *stream);

/*
 * dL/dA on A's pattern: d_grad_vals[k] = -lambda[row(k)] * x[col(k)] for every
 * stored scalar k (the last step of the adjoint, on its own).  Asynchronous.
 */
sla_status sla_pattern_grad(sla_mat_t A, const void *d_lambda, const void *d_x,
                            void *d_grad_vals, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 *
 * sla_init() prepares the CURRENT device once: it resolves the device
 * address of the library's fixed solver scratch (32 MiB, a static device
 * array that every device the library runs on holds until the process
 * ends) and reserves a pinned polling record.  It may allocate (pinned
 * host memory, events) and must run outside the allocation-free region.
 * Idempotent; SLA_ERR_HIP if the device cannot be queried.
 *
 * sla_pcg_solve_noalloc() is sla_pcg_solve with its workspace taken from
 * that scratch: it calls no hipMalloc, hipFree, hipHostMalloc or other
 * allocating routine.  Same arguments (minus the workspace), iteration,
 * stopping rule, statuses and results as sla_pcg_solve, except that it
 * always runs in A's own row order (no locality ordering, which would build
 * permuted copies; results agree to rounding) and records no profiling
 * events.  A and G must belong to the current device.  Errors:
 * SLA_ERR_INVALID_ARG if sla_init() has not run on the current device or
 * the system's workspace (sla_pcg_workspace_size without the ordering's two
 * extra vectors) exceeds 32 MiB -- about 500k rows in fp64 -- plus every
 * error of sla_pcg_solve.  All calls on one device share the one scratch
 * array, which keeps the last call's contents (the solve clears what must
 * start at zero); the library serialises calls from different host threads
 * on the same device, so overlapping calls wait rather than race.
 * Synchronous like sla_pcg_solve.
 */
sla_status sla_init(void);
sla_status sla_pcg_solve_noalloc(sla_mat_t A, sla_mat_t G, double eps, const void *d_b,
                                 void *d_x, double rtol, int32_t maxit, void *stream,
                                 sla_solve_info *info);

/* Human-readable name of a status, and the calling thread's last error text. */
const char *sla_status_string(sla_status st);
const char *sla_last_error(void);

/*
 * Kernel timing with HIP events recorded on the caller's stream around each
 * launch of the solver's kernels.  `enable` is a bit mask of kernel classes
 * (bit c records class c; 0 = off, the default).  Only launches that did work
 * are counted (not the no-op launches after convergence).  Classes:
 * 0 = A product step (q = A p, fused p and x updates, p.q), 1 = G^T product
 * step (fused residual update, ||r||^2), 2 = G product step (z = G t + eps r,
 * r.z), 3 = plain sla_spmv.  sla_get_profile returns the launch count and the
 * summed event time (ms) of a class since the last sla_reset_profile.
 */
sla_status sla_set_profiling(int32_t enable);
/*
 * Sampling of the solver's kernel timing: events bracket only the launches of
 * iterations k with k % every == 0 (the start-up launches, k = 0, always).
 * every = 1 (the default) times every launch; a larger stride keeps the
 * event packets from slowing the solve they measure.  Applies to classes
 * 0-2; plain sla_spmv calls are always timed when class 3 is enabled.
 * Error: SLA_ERR_INVALID_ARG if every < 1.
 */
sla_status sla_set_profiling_stride(int32_t every);
sla_status sla_get_profile(int32_t kernel_class, int64_t *launches, double *total_ms);
sla_status sla_reset_profile(void);

#ifdef __cplusplus
}
#endif

#endif /* SLA_H */
