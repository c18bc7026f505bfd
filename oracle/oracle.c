/*
 * oracle.c -- plain CPU reference for preconditioned conjugate gradients with a
 * factorised sparse approximate inverse, and for the adjoint of that solve.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity oracle that the tests,
 * the smoke check and the benchmark's CPU-baseline leg compare the HIP library
 * against.  The product (the HIP library and its Python binding) never links,
 * loads or calls it, and it shares no code with the product.
 *
 * Everything is fp64, evaluated in the order written (build with
 * -ffp-contract=off so no fused multiply-adds appear).  Loops over rows may run
 * under OpenMP; every row is computed by one thread in storage order and every
 * dot product is summed in fixed blocks of ORC_DOT_BLOCK elements whose
 * partial sums are added in block order, so the result is bitwise identical
 * for any thread count.
 *
 * Sources (pages, as cited):
 *  - "Learning Sparse Approximate Inverse Preconditioners for Conjugate Gradient
 *    Solvers on GPUs", section "Approach": the preconditioner is
 *    M^-1 = G G^T + eps I with G on A's sparsity, so applying it costs two
 *    sparse matrix-vector products; CG is used on sparse SPD systems
 *    ("Problem").
 *  - "torch-sla: Differentiable Sparse Linear Algebra ...", Technical Summary,
 *    Methodology 2 "Adjoint Differentiation Framework", linear systems: for
 *    A x = b the backward pass solves A^T lambda = dL/dx once and the matrix
 *    gradient is -lambda_i x_j on the sparsity pattern only; memory is
 *    O(n + nnz) independent of the iteration count.
 *  - CG itself is the textbook preconditioned conjugate-gradient iteration
 *    (Hestenes-Stiefel with a symmetric positive-definite preconditioner).
 *
 * Readings where the pages are silent (listed in the design notes too):
 *  - stopping rule: recursive residual ||r_k||_2 <= rtol ||b||_2, x_0 = 0,
 *    tested right after the residual update and before the preconditioner;
 *  - iteration count = number of products with A = number of x updates;
 *  - ||b|| = 0 returns x = 0 after 0 iterations (converged); maxit = 0 with
 *    b != 0 returns x = 0, not converged;
 *  - breakdown (p.Ap <= 0, r.z <= 0, or a non-finite scalar) is an error;
 *  - G's pattern is the lower triangle of A's (block-lower for BSR);
 *  - the adjoint reuses the same G, eps, rtol and maxit, and A^T = A for the
 *    SPD matrices the method targets is used as is (the transposed solve is
 *    the same solve); dL/db = lambda.
 *
 * Matrices are square BSR with block size bs (bs = 1 is CSR): row_ptr has
 * nbr + 1 entries, col[] block columns ascending within a row, val[] has
 * bs*bs values per stored block, row-major inside the block.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_DOT_BLOCK 4096

enum {
    ORC_OK = 0,
    ORC_NOT_CONVERGED = 1,
    ORC_ERR_ARG = -1,
    ORC_ERR_BREAKDOWN = -3,
    ORC_ERR_NONFINITE = -4,
    ORC_ERR_NOMEM = -6
};

/* Summation order of long rows.  0 (the oracle): every row sum starts at
 * 0.0 and adds val*x in storage order.  A build with ORC_ROW_CHUNK = c > 0
 * instead sums each row longer than c / 2 entries in consecutive chunks of c
 * entries (each from 0.0, in storage order) and adds the chunk sums in
 * order: another valid rounding order of the same sum, used only to measure
 * how far the solver's stopping iteration moves with the summation order on
 * systems with very long rows. */
#ifndef ORC_ROW_CHUNK
#define ORC_ROW_CHUNK 0
#endif

/* y = A x.  Row sums start at 0.0 and add val*x in storage order
 * (the definition of a sparse matrix-vector product). */
void orc_spmv(int64_t nbr, int bs, const int32_t *row_ptr, const int32_t *col,
              const double *val, const double *x, double *y)
{
    const int64_t bb = (int64_t)bs * bs;
#pragma omp parallel for schedule(static)
    for (int64_t I = 0; I < nbr; ++I) {
        const int64_t kb = row_ptr[I], ke = row_ptr[I + 1];
        const int chunked = ORC_ROW_CHUNK > 0 && 2 * (ke - kb) > (int64_t)ORC_ROW_CHUNK;
        for (int r = 0; r < bs; ++r) {
            double s = 0.0, done = 0.0;
            for (int64_t k = kb; k < ke; ++k) {
                if (chunked && k > kb && (k - kb) % (ORC_ROW_CHUNK > 0 ? ORC_ROW_CHUNK : 1) == 0) {
                    done += s;
                    s = 0.0;
                }
                const int64_t J = col[k];
                const double *blk = val + k * bb + (int64_t)r * bs;
                for (int c = 0; c < bs; ++c)
                    s += blk[c] * x[J * bs + c];
            }
            y[I * bs + r] = chunked ? done + s : s;
        }
    }
}

/* Transpose of a square BSR matrix: count entries per block column, prefix
 * sum, then place entries while walking rows in order, so every row of the
 * result lists its columns ascending.  Blocks are transposed as well. */
int orc_transpose(int64_t nbr, int bs, const int32_t *row_ptr, const int32_t *col,
                  const double *val, int32_t *t_row_ptr, int32_t *t_col, double *t_val)
{
    const int64_t bb = (int64_t)bs * bs;
    const int64_t nnzb = row_ptr[nbr];
    int64_t *next = (int64_t *)calloc((size_t)nbr + 1, sizeof(int64_t));
    if (!next) return ORC_ERR_NOMEM;
    for (int64_t k = 0; k < nnzb; ++k) next[col[k] + 1] += 1;
    for (int64_t j = 0; j < nbr; ++j) next[j + 1] += next[j];
    for (int64_t j = 0; j <= nbr; ++j) t_row_ptr[j] = (int32_t)next[j];
    for (int64_t I = 0; I < nbr; ++I) {
        for (int64_t k = row_ptr[I]; k < row_ptr[I + 1]; ++k) {
            const int64_t J = col[k];
            const int64_t dst = next[J]++;
            t_col[dst] = (int32_t)I;
            for (int r = 0; r < bs; ++r)
                for (int c = 0; c < bs; ++c)
                    t_val[dst * bb + (int64_t)c * bs + r] = val[k * bb + (int64_t)r * bs + c];
        }
    }
    free(next);
    return ORC_OK;
}

/* a . b, summed in fixed blocks. */
double orc_dot(int64_t n, const double *a, const double *b)
{
    const int64_t nblk = (n + ORC_DOT_BLOCK - 1) / ORC_DOT_BLOCK;
    double *part = (double *)malloc((size_t)(nblk > 0 ? nblk : 1) * sizeof(double));
    if (!part) return NAN;
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < nblk; ++q) {
        const int64_t lo = q * ORC_DOT_BLOCK;
        const int64_t hi = (lo + ORC_DOT_BLOCK < n) ? lo + ORC_DOT_BLOCK : n;
        double s = 0.0;
        for (int64_t i = lo; i < hi; ++i) s += a[i] * b[i];
        part[q] = s;
    }
    double s = 0.0;
    for (int64_t q = 0; q < nblk; ++q) s += part[q];
    free(part);
    return s;
}

typedef struct {
    int64_t nbr;
    int bs;
    const int32_t *row_ptr;
    const int32_t *col;
    const double *val;
} orc_mat;

/* z = G (G^T r) + eps r, with G^T given explicitly (t is scratch). */
static void precond_apply(const orc_mat *G, const orc_mat *Gt, double eps, const double *r,
                          double *t, double *z, int64_t n)
{
    orc_spmv(Gt->nbr, Gt->bs, Gt->row_ptr, Gt->col, Gt->val, r, t);
    orc_spmv(G->nbr, G->bs, G->row_ptr, G->col, G->val, t, z);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) z[i] = z[i] + eps * r[i];
}

/* Exported for the tests: z = (G G^T + eps I) r. */
int orc_precond_apply(int64_t nbr, int bs, const int32_t *g_row_ptr, const int32_t *g_col,
                      const double *g_val, double eps, const double *r, double *z)
{
    const int64_t n = nbr * bs;
    const int64_t nnzb = g_row_ptr[nbr];
    const int64_t bb = (int64_t)bs * bs;
    int32_t *trp = (int32_t *)malloc(((size_t)nbr + 1) * sizeof(int32_t));
    int32_t *tci = (int32_t *)malloc((size_t)(nnzb > 0 ? nnzb : 1) * sizeof(int32_t));
    double *tv = (double *)malloc((size_t)(nnzb > 0 ? nnzb * bb : 1) * sizeof(double));
    double *t = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    int st = ORC_OK;
    if (!trp || !tci || !tv || !t) { st = ORC_ERR_NOMEM; goto out; }
    orc_transpose(nbr, bs, g_row_ptr, g_col, g_val, trp, tci, tv);
    {
        orc_mat G = {nbr, bs, g_row_ptr, g_col, g_val};
        orc_mat Gt = {nbr, bs, trp, tci, tv};
        precond_apply(&G, &Gt, eps, r, t, z, n);
    }
out:
    free(trp); free(tci); free(tv); free(t);
    return st;
}

/* Preconditioned CG for A x = b with M^-1 = G G^T + eps I.
 * On return: x = last iterate, *iters = number of A-products, *relres =
 * ||r_k|| / ||b|| of the recursive residual (0 when b = 0).
 * When hist_len > 0 the step lengths are recorded as hist_a[k-1] = alpha_k and
 * the direction coefficients as hist_b[k-1] = beta_k = rho_k / rho_{k-1}, for
 * every k <= hist_len that the iteration reaches. */
int orc_pcg_history(int64_t nbr, int bs,
                    const int32_t *a_row_ptr, const int32_t *a_col, const double *a_val,
                    const int32_t *g_row_ptr, const int32_t *g_col, const double *g_val,
                    double eps, const double *b, double *x, double rtol, int32_t maxit,
                    int32_t *iters, double *relres, double *hist_a, double *hist_b,
                    int32_t hist_len)
{
    const int64_t n = nbr * bs;
    const int64_t bb = (int64_t)bs * bs;
    const int64_t gnnzb = g_row_ptr[nbr];
    *iters = 0;
    *relres = 0.0;
    if (nbr < 0 || bs < 1 || maxit < 0 || !(rtol >= 0.0) || !(eps >= 0.0)) return ORC_ERR_ARG;

    int32_t *trp = (int32_t *)malloc(((size_t)nbr + 1) * sizeof(int32_t));
    int32_t *tci = (int32_t *)malloc((size_t)(gnnzb > 0 ? gnnzb : 1) * sizeof(int32_t));
    double *tv = (double *)malloc((size_t)(gnnzb > 0 ? gnnzb * bb : 1) * sizeof(double));
    const size_t vb = (size_t)(n > 0 ? n : 1) * sizeof(double);
    double *r = (double *)malloc(vb), *z = (double *)malloc(vb), *p = (double *)malloc(vb);
    double *q = (double *)malloc(vb), *t = (double *)malloc(vb);
    int st = ORC_OK;
    if (!trp || !tci || !tv || !r || !z || !p || !q || !t) { st = ORC_ERR_NOMEM; goto out; }

    orc_transpose(nbr, bs, g_row_ptr, g_col, g_val, trp, tci, tv);
    {
        const orc_mat A = {nbr, bs, a_row_ptr, a_col, a_val};
        const orc_mat G = {nbr, bs, g_row_ptr, g_col, g_val};
        const orc_mat Gt = {nbr, bs, trp, tci, tv};

        for (int64_t i = 0; i < n; ++i) { x[i] = 0.0; r[i] = b[i]; }
        const double bnorm = sqrt(orc_dot(n, b, b));
        if (!isfinite(bnorm)) { st = ORC_ERR_NONFINITE; goto out; }
        if (bnorm == 0.0) { st = ORC_OK; goto out; }
        if (maxit == 0) { *relres = 1.0; st = ORC_NOT_CONVERGED; goto out; }

        precond_apply(&G, &Gt, eps, r, t, z, n);
        double rho = orc_dot(n, r, z);
        if (!(rho > 0.0) || !isfinite(rho)) { st = ORC_ERR_BREAKDOWN; goto out; }
        for (int64_t i = 0; i < n; ++i) p[i] = z[i];

        for (int32_t k = 1; k <= maxit; ++k) {
            orc_spmv(A.nbr, A.bs, A.row_ptr, A.col, A.val, p, q);
            const double sigma = orc_dot(n, p, q);
            if (!(sigma > 0.0) || !isfinite(sigma)) { *iters = k - 1; st = ORC_ERR_BREAKDOWN; goto out; }
            const double alpha = rho / sigma;
            if (k <= hist_len) hist_a[k - 1] = alpha;
#pragma omp parallel for schedule(static)
            for (int64_t i = 0; i < n; ++i) {
                x[i] = x[i] + alpha * p[i];
                r[i] = r[i] - alpha * q[i];
            }
            *iters = k;
            const double rnorm = sqrt(orc_dot(n, r, r));
            *relres = rnorm / bnorm;
            if (!isfinite(rnorm)) { st = ORC_ERR_BREAKDOWN; goto out; }
            if (rnorm <= rtol * bnorm) { st = ORC_OK; goto out; }
            if (k == maxit) break;
            precond_apply(&G, &Gt, eps, r, t, z, n);
            const double rho_new = orc_dot(n, r, z);
            if (!(rho_new > 0.0) || !isfinite(rho_new)) { st = ORC_ERR_BREAKDOWN; goto out; }
            const double beta = rho_new / rho;
            if (k <= hist_len) hist_b[k - 1] = beta;
#pragma omp parallel for schedule(static)
            for (int64_t i = 0; i < n; ++i) p[i] = z[i] + beta * p[i];
            rho = rho_new;
        }
        st = ORC_NOT_CONVERGED;
    }
out:
    free(trp); free(tci); free(tv);
    free(r); free(z); free(p); free(q); free(t);
    return st;
}

int orc_pcg(int64_t nbr, int bs,
            const int32_t *a_row_ptr, const int32_t *a_col, const double *a_val,
            const int32_t *g_row_ptr, const int32_t *g_col, const double *g_val,
            double eps, const double *b, double *x, double rtol, int32_t maxit,
            int32_t *iters, double *relres)
{
    return orc_pcg_history(nbr, bs, a_row_ptr, a_col, a_val, g_row_ptr, g_col, g_val, eps, b,
                           x, rtol, maxit, iters, relres, NULL, NULL, 0);
}

/* The Lanczos tridiagonal T_k of the preconditioned operator M^-1 A that k
 * steps of PCG implicitly build (the CG-Lanczos connection of textbook
 * iterative-methods theory; its eigenvalues are Ritz values of M^-1 A):
 *   T_11 = 1 / alpha_1,
 *   T_jj = 1 / alpha_j + beta_{j-1} / alpha_{j-1}          (j = 2 .. k),
 *   T_j,j+1 = T_j+1,j = sqrt(beta_j) / alpha_j             (j = 1 .. k-1).
 * diag gets k entries, off gets k-1. */
int orc_lanczos_tridiag(const double *alpha, const double *beta, int32_t k, double *diag,
                        double *off)
{
    if (k < 1) return ORC_ERR_ARG;
    for (int32_t j = 0; j < k; ++j) {
        if (!(alpha[j] > 0.0) || !isfinite(alpha[j])) return ORC_ERR_ARG;
        if (j + 1 < k && (!(beta[j] >= 0.0) || !isfinite(beta[j]))) return ORC_ERR_ARG;
    }
    for (int32_t j = 0; j < k; ++j) {
        diag[j] = 1.0 / alpha[j];
        if (j > 0) diag[j] = diag[j] + beta[j - 1] / alpha[j - 1];
        if (j + 1 < k) off[j] = sqrt(beta[j]) / alpha[j];
    }
    return ORC_OK;
}

/* Stochastic estimate of the scale-invariant SAI loss || A M^-1 / s - I ||_F^2
 * ("Learning Sparse Approximate Inverse Preconditioners ...", Approach):
 * for probe vectors w_j (column j of the n x nprobe column-major array w),
 * out[j] = || A (M^-1 w_j) / s - w_j ||^2, with M^-1 w = G (G^T w) + eps w.
 * For probes with E[w w^T] = I the mean of out is an unbiased estimate of the
 * loss; with the n unit vectors as probes their sum is the loss exactly. */
int orc_sai_loss(int64_t nbr, int bs,
                 const int32_t *a_row_ptr, const int32_t *a_col, const double *a_val,
                 const int32_t *g_row_ptr, const int32_t *g_col, const double *g_val,
                 double eps, const double *w, int32_t nprobe, double s, double *out)
{
    const int64_t n = nbr * bs;
    if (nbr < 0 || bs < 1 || nprobe < 0 || !(eps >= 0.0) || !(s > 0.0) || !isfinite(s))
        return ORC_ERR_ARG;
    const size_t vb = (size_t)(n > 0 ? n : 1) * sizeof(double);
    double *z = (double *)malloc(vb), *y = (double *)malloc(vb), *d = (double *)malloc(vb);
    int st = ORC_OK;
    if (!z || !y || !d) { st = ORC_ERR_NOMEM; goto out; }
    for (int32_t j = 0; j < nprobe; ++j) {
        const double *wj = w + (int64_t)j * n;
        st = orc_precond_apply(nbr, bs, g_row_ptr, g_col, g_val, eps, wj, z);
        if (st != ORC_OK) goto out;
        orc_spmv(nbr, bs, a_row_ptr, a_col, a_val, z, y);
        for (int64_t i = 0; i < n; ++i) d[i] = y[i] / s - wj[i];
        out[j] = orc_dot(n, d, d);
    }
out:
    free(z); free(y); free(d);
    return st;
}

/* dL/dA on A's pattern: for every stored scalar (i, j), -lambda_i x_j,
 * written in A's storage order (block by block, row-major inside a block). */
void orc_pattern_grad(int64_t nbr, int bs, const int32_t *a_row_ptr, const int32_t *a_col,
                      const double *lam, const double *x, double *grad_val)
{
    const int64_t bb = (int64_t)bs * bs;
#pragma omp parallel for schedule(static)
    for (int64_t I = 0; I < nbr; ++I) {
        for (int64_t k = a_row_ptr[I]; k < a_row_ptr[I + 1]; ++k) {
            const int64_t J = a_col[k];
            for (int r = 0; r < bs; ++r)
                for (int c = 0; c < bs; ++c)
                    grad_val[k * bb + (int64_t)r * bs + c] = -(lam[I * bs + r] * x[J * bs + c]);
        }
    }
}

/* Adjoint of x = A^-1 b for a loss L(x) with gradient gx = dL/dx:
 * lambda solves A^T lambda = gx (A^T = A here), dL/db = lambda, and
 * dL/dA at every stored scalar (i, j) is -lambda_i x_j, in A's storage order. */
int orc_adjoint(int64_t nbr, int bs,
                const int32_t *a_row_ptr, const int32_t *a_col, const double *a_val,
                const int32_t *g_row_ptr, const int32_t *g_col, const double *g_val,
                double eps, const double *x, const double *gx, double *lam, double *grad_val,
                double rtol, int32_t maxit, int32_t *iters, double *relres)
{
    int st = orc_pcg(nbr, bs, a_row_ptr, a_col, a_val, g_row_ptr, g_col, g_val, eps, gx, lam,
                     rtol, maxit, iters, relres);
    if (st < 0) return st;
    orc_pattern_grad(nbr, bs, a_row_ptr, a_col, lam, x, grad_val);
    return st;
}

/* Several right-hand sides sharing A and G.  b and x are n x k and row-major:
 * b[i * k + j] is entry i of right-hand side j.  Every column is its own PCG
 * solve (the k solves share only the operators), with its own iteration count,
 * residual and status in iters[j], relres[j], status[j].  Returns the first
 * negative column status, else ORC_NOT_CONVERGED if any column did not
 * converge, else ORC_OK. */
int orc_pcg_multi(int64_t nbr, int bs,
                  const int32_t *a_row_ptr, const int32_t *a_col, const double *a_val,
                  const int32_t *g_row_ptr, const int32_t *g_col, const double *g_val,
                  double eps, const double *b, double *x, int32_t k, double rtol, int32_t maxit,
                  int32_t *iters, double *relres, int32_t *status)
{
    const int64_t n = nbr * bs;
    if (nbr < 0 || bs < 1 || k < 1) return ORC_ERR_ARG;
    const size_t vb = (size_t)(n > 0 ? n : 1) * sizeof(double);
    double *bj = (double *)malloc(vb), *xj = (double *)malloc(vb);
    int ret = ORC_OK;
    if (!bj || !xj) { ret = ORC_ERR_NOMEM; goto out; }
    for (int32_t j = 0; j < k; ++j) {
        for (int64_t i = 0; i < n; ++i) bj[i] = b[i * k + j];
        status[j] = orc_pcg(nbr, bs, a_row_ptr, a_col, a_val, g_row_ptr, g_col, g_val, eps, bj,
                            xj, rtol, maxit, &iters[j], &relres[j]);
        for (int64_t i = 0; i < n; ++i) x[i * k + j] = xj[i];
        if (status[j] < 0 && ret >= 0) ret = status[j];
        else if (status[j] == ORC_NOT_CONVERGED && ret == ORC_OK) ret = ORC_NOT_CONVERGED;
    }
out:
    free(bj); free(xj);
    return ret;
}

/* Adjoint of k solves X = A^-1 B sharing A, for a loss L(X) with gradient
 * gx = dL/dX (n x k, row-major like x): column j of lam solves
 * A^T lam_j = gx_j, dL/dB = lam, and since every solve uses the same A, its
 * gradient is the sum over the solves of -lam_j[i] x_j[c] at every stored
 * scalar (i, c), accumulated over j = 0 .. k-1 in that order. */
int orc_adjoint_multi(int64_t nbr, int bs,
                      const int32_t *a_row_ptr, const int32_t *a_col, const double *a_val,
                      const int32_t *g_row_ptr, const int32_t *g_col, const double *g_val,
                      double eps, const double *x, const double *gx, double *lam,
                      double *grad_val, int32_t k, double rtol, int32_t maxit, int32_t *iters,
                      double *relres, int32_t *status)
{
    const int64_t n = nbr * bs;
    const int64_t bb = (int64_t)bs * bs;
    if (nbr < 0 || bs < 1 || k < 1) return ORC_ERR_ARG;
    int ret = orc_pcg_multi(nbr, bs, a_row_ptr, a_col, a_val, g_row_ptr, g_col, g_val, eps, gx,
                            lam, k, rtol, maxit, iters, relres, status);
    if (ret < 0) return ret;
    (void)n;
#pragma omp parallel for schedule(static)
    for (int64_t I = 0; I < nbr; ++I) {
        for (int64_t e = a_row_ptr[I]; e < a_row_ptr[I + 1]; ++e) {
            const int64_t J = a_col[e];
            for (int r = 0; r < bs; ++r)
                for (int c = 0; c < bs; ++c) {
                    double g = 0.0;
                    for (int32_t j = 0; j < k; ++j)
                        g = g - lam[(I * bs + r) * k + j] * x[(J * bs + c) * k + j];
                    grad_val[e * bb + (int64_t)r * bs + c] = g;
                }
        }
    }
    return ret;
}

int orc_dot_block(void) { return ORC_DOT_BLOCK; }

/* Threads the OpenMP row loops use (1 when built without OpenMP), and a
 * setter for timing runs (results are bitwise the same for any count). */
#ifdef _OPENMP
#include <omp.h>
int orc_num_threads(void) { return omp_get_max_threads(); }
void orc_set_num_threads(int t) { omp_set_num_threads(t > 0 ? t : 1); }
#else
int orc_num_threads(void) { return 1; }
void orc_set_num_threads(int t) { (void)t; }
#endif
