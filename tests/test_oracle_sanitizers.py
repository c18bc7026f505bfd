"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
a C driver calls every oracle entry point on small CSR and 3x3-BSR systems,
including the empty system, b = 0, maxit = 0 and a history buffer shorter
than the iteration count, in a build with -fsanitize=address,undefined; any
out-of-bounds access, leak or undefined operation fails the run."""
import os
import shutil
import subprocess

import pytest

import oracle

DRIVER = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_spmv(int64_t, int, const int32_t*, const int32_t*, const double*, const double*, double*);
int orc_transpose(int64_t, int, const int32_t*, const int32_t*, const double*, int32_t*, int32_t*,
                  double*);
double orc_dot(int64_t, const double*, const double*);
int orc_precond_apply(int64_t, int, const int32_t*, const int32_t*, const double*, double,
                      const double*, double*);
int orc_pcg(int64_t, int, const int32_t*, const int32_t*, const double*, const int32_t*,
            const int32_t*, const double*, double, const double*, double*, double, int32_t,
            int32_t*, double*);
int orc_pcg_history(int64_t, int, const int32_t*, const int32_t*, const double*, const int32_t*,
                    const int32_t*, const double*, double, const double*, double*, double,
                    int32_t, int32_t*, double*, double*, double*, int32_t);
int orc_lanczos_tridiag(const double*, const double*, int32_t, double*, double*);
int orc_sai_loss(int64_t, int, const int32_t*, const int32_t*, const double*, const int32_t*,
                 const int32_t*, const double*, double, const double*, int32_t, double, double*);
void orc_pattern_grad(int64_t, int, const int32_t*, const int32_t*, const double*, const double*,
                      double*);
int orc_adjoint(int64_t, int, const int32_t*, const int32_t*, const double*, const int32_t*,
                const int32_t*, const double*, double, const double*, const double*, double*,
                double*, double, int32_t, int32_t*, double*);
int orc_pcg_multi(int64_t, int, const int32_t*, const int32_t*, const double*, const int32_t*,
                  const int32_t*, const double*, double, const double*, double*, int32_t, double,
                  int32_t, int32_t*, double*, int32_t*);
int orc_adjoint_multi(int64_t, int, const int32_t*, const int32_t*, const double*,
                      const int32_t*, const int32_t*, const double*, double, const double*,
                      const double*, double*, double*, int32_t, double, int32_t, int32_t*,
                      double*, int32_t*);

typedef struct { int64_t nbr; int bs; int32_t *rp, *ci; double *v; } Mat;

/* block tridiagonal: diagonal blocks d*I + 0.1*(1 on the off-diagonals), off blocks -I */
static Mat tri(int64_t nbr, int bs, double d, int lower_only, double off) {
  Mat m = {nbr, bs, malloc(sizeof(int32_t) * (nbr + 1)), malloc(sizeof(int32_t) * 3 * nbr + 4),
           malloc(sizeof(double) * 3 * nbr * bs * bs + 8)};
  int64_t k = 0;
  for (int64_t i = 0; i < nbr; ++i) {
    m.rp[i] = (int32_t)k;
    for (int64_t j = i - 1; j <= i + 1; ++j) {
      if (j < 0 || j >= nbr || (lower_only && j > i)) continue;
      m.ci[k] = (int32_t)j;
      for (int r = 0; r < bs; ++r)
        for (int c = 0; c < bs; ++c) {
          double v = 0.0;
          if (j == i) v = (r == c) ? d : (lower_only ? 0.0 : 0.1);
          else v = (r == c) ? off : 0.0;
          m.v[k * bs * bs + r * bs + c] = v;
        }
      ++k;
    }
  }
  m.rp[nbr] = (int32_t)k;
  return m;
}

static void drop(Mat m) { free(m.rp); free(m.ci); free(m.v); }

static int run(int64_t nbr, int bs) {
  Mat A = tri(nbr, bs, 4.0, 0, -1.0), G = tri(nbr, bs, 0.5, 1, 0.05);
  const int64_t n = nbr * bs, nnz = (int64_t)A.rp[nbr] * bs * bs;
  const int k = 3;
  double *b = calloc(n * k + 1, 8), *x = calloc(n * k + 1, 8), *y = calloc(n + 1, 8);
  double *lam = calloc(n * k + 1, 8), *gv = calloc(nnz + 1, 8), *ha = calloc(4, 8);
  double *hb = calloc(4, 8), *d = calloc(4, 8), *e = calloc(4, 8), *out = calloc(k, 8);
  double *rr = calloc(k, 8);
  int32_t *its = calloc(k, 4), *sts = calloc(k, 4);
  int32_t *trp = malloc(4 * (nbr + 1)), *tci = malloc(4 * (G.rp[nbr] + 1));
  double *tv = malloc(8 * ((int64_t)G.rp[nbr] * bs * bs + 1));
  for (int64_t i = 0; i < n * k; ++i) b[i] = sin(0.37 * (double)i + 0.1);
  int32_t it = 0;
  double rel = 0.0;
  int fails = 0;
  orc_spmv(nbr, bs, A.rp, A.ci, A.v, b, y);
  fails += orc_transpose(nbr, bs, G.rp, G.ci, G.v, trp, tci, tv) != 0;
  (void)orc_dot(n, b, y);
  fails += orc_precond_apply(nbr, bs, G.rp, G.ci, G.v, 3e-3, b, y) != 0;
  int st = orc_pcg(nbr, bs, A.rp, A.ci, A.v, G.rp, G.ci, G.v, 3e-3, b, x, 1e-10, 500, &it, &rel);
  fails += !(st == 0 || (n == 0 && st == 0));
  /* history shorter than the iterations */
  st = orc_pcg_history(nbr, bs, A.rp, A.ci, A.v, G.rp, G.ci, G.v, 3e-3, b, x, 1e-10, 500, &it,
                       &rel, ha, hb, 4);
  if (n > 0 && it >= 2) fails += orc_lanczos_tridiag(ha, hb, it < 4 ? it : 4, d, e) != 0;
  fails += orc_sai_loss(nbr, bs, A.rp, A.ci, A.v, G.rp, G.ci, G.v, 3e-3, b, k, 2.0, out) != 0;
  orc_pattern_grad(nbr, bs, A.rp, A.ci, y, x, gv);
  st = orc_adjoint(nbr, bs, A.rp, A.ci, A.v, G.rp, G.ci, G.v, 3e-3, x, b, lam, gv, 1e-10, 500,
                   &it, &rel);
  fails += st != 0;
  st = orc_pcg_multi(nbr, bs, A.rp, A.ci, A.v, G.rp, G.ci, G.v, 3e-3, b, x, k, 1e-10, 500, its,
                     rr, sts);
  fails += st != 0;
  st = orc_adjoint_multi(nbr, bs, A.rp, A.ci, A.v, G.rp, G.ci, G.v, 3e-3, x, b, lam, gv, k,
                         1e-10, 500, its, rr, sts);
  fails += st != 0;
  /* b = 0 (converged at once) and maxit = 0 */
  memset(b, 0, 8 * (n + 1));
  st = orc_pcg(nbr, bs, A.rp, A.ci, A.v, G.rp, G.ci, G.v, 3e-3, b, x, 1e-10, 500, &it, &rel);
  fails += st != 0 || it != 0;
  b[0] = 1.0;
  st = orc_pcg(nbr, bs, A.rp, A.ci, A.v, G.rp, G.ci, G.v, 3e-3, b, x, 1e-10, 0, &it, &rel);
  fails += n > 0 ? (st != 1 || it != 0) : (st != 0);
  free(b); free(x); free(y); free(lam); free(gv); free(ha); free(hb); free(d); free(e);
  free(out); free(rr); free(its); free(sts); free(trp); free(tci); free(tv);
  drop(A); drop(G);
  if (fails) printf("failures at nbr=%lld bs=%d: %d\n", (long long)nbr, bs, fails);
  return fails;
}

int main(void) {
  int f = run(37, 1) + run(12, 3) + run(1, 1) + run(0, 1) + run(4500, 1);
  printf(f ? "FAILED\n" : "ok\n");
  return f != 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    exe = tmp_path / "oracle_asan"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-ffp-contract=off", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", str(drv), oracle.SRC, "-o", str(exe), "-lm"],
                   check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    out = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), out.stdout + out.stderr
