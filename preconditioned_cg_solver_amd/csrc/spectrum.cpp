// Extreme eigenvalues of the Lanczos tridiagonal that preconditioned CG builds
// implicitly (the CG-Lanczos connection): with CG's step lengths alpha_j and
// direction coefficients beta_j = rho_j / rho_{j-1},
//   T_jj = 1/alpha_j + beta_{j-1}/alpha_{j-1},   T_j,j+1 = sqrt(beta_j)/alpha_j,
// and the eigenvalues of T_k are Ritz values of M^-1 A, so their extremes
// bracket the preconditioned spectrum from inside and kappa(M^-1 A) is
// estimated by lmax / lmin.  The condition number is one of the metrics of
// "Learning Sparse Approximate Inverse Preconditioners for Conjugate Gradient
// Solvers on GPUs" (Experimental setup).
//
// Host code: k is at most the iteration count, so T_k is tiny next to the
// solve.  The extremes come from Sturm-sequence bisection (the number of
// negative pivots of the LDL^T factorisation of T - x I counts the eigenvalues
// below x), started from the Gershgorin interval.

#include <cmath>
#include <limits>
#include <vector>

#include "internal.h"

namespace sla {
namespace {

// Number of eigenvalues of the symmetric tridiagonal (d, e2 = e^2) below x.
int count_below(const std::vector<double>& d, const std::vector<double>& e2, double x,
                double tiny) {
  int c = 0;
  double q = 1.0;
  for (size_t i = 0; i < d.size(); ++i) {
    q = d[i] - x - (i > 0 ? e2[i - 1] / q : 0.0);
    if (q == 0.0) q = -tiny;  // a zero pivot counts as negative, nudged off zero
    if (q < 0.0) ++c;
  }
  return c;
}

// The m-th smallest eigenvalue (0-based) by bisection on [lo, hi].
double bisect(const std::vector<double>& d, const std::vector<double>& e2, int m, double lo,
              double hi, double tiny) {
  for (int it = 0; it < 200; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;  // interval down to adjacent doubles
    if (count_below(d, e2, mid, tiny) > m) hi = mid;
    else lo = mid;
  }
  return 0.5 * (lo + hi);
}

}  // namespace

sla_status lanczos_extremes(const double* alpha, const double* beta, int32_t k, double* lmin,
                            double* lmax) {
  std::vector<double> d(k), e2(k > 1 ? k - 1 : 0);
  for (int32_t j = 0; j < k; ++j) {
    if (!(alpha[j] > 0.0) || !std::isfinite(alpha[j])) {
      set_error("alpha must be finite and > 0");
      return SLA_ERR_INVALID_ARG;
    }
    if (j + 1 < k && (!(beta[j] >= 0.0) || !std::isfinite(beta[j]))) {
      set_error("beta must be finite and >= 0");
      return SLA_ERR_INVALID_ARG;
    }
  }
  for (int32_t j = 0; j < k; ++j) {
    d[j] = 1.0 / alpha[j] + (j > 0 ? beta[j - 1] / alpha[j - 1] : 0.0);
    if (j + 1 < k) e2[j] = beta[j] / (alpha[j] * alpha[j]);
  }
  double lo = std::numeric_limits<double>::infinity(), hi = -lo, scale = 0.0;
  for (int32_t j = 0; j < k; ++j) {
    const double r = (j > 0 ? std::sqrt(e2[j - 1]) : 0.0) + (j + 1 < k ? std::sqrt(e2[j]) : 0.0);
    lo = std::min(lo, d[j] - r);
    hi = std::max(hi, d[j] + r);
    scale = std::max(scale, std::fabs(d[j]) + r);
  }
  if (!std::isfinite(lo) || !std::isfinite(hi)) {
    set_error("tridiagonal entries overflow");
    return SLA_ERR_INVALID_ARG;
  }
  const double pad = 4.0 * std::numeric_limits<double>::epsilon() * scale;
  lo -= pad;
  hi += pad;
  const double tiny = std::numeric_limits<double>::min() / std::numeric_limits<double>::epsilon();
  *lmin = bisect(d, e2, 0, lo, hi, tiny);
  *lmax = bisect(d, e2, k - 1, lo, hi, tiny);
  return SLA_OK;
}

}  // namespace sla
