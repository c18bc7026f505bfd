// Host-side schedule of the PCG driver's batches of iterations (plain C++,
// no HIP: the host tests compile it on its own).
#pragma once

#include <algorithm>
#include <cmath>

namespace sla {

// Sizes the host's batches of iterations.  Full batches of `full` until the
// polled residuals predict the stopping iteration: a geometric fit of
// ||r||^2 between the last two polls (one poll is not enough: CG's first
// iterations often drop the residual faster than the rest do).  Then only
// the iterations up to the prediction plus a margin that grows with the
// distance, so that few launches run after convergence (they return at once
// but each costs a dispatch).  A record past a predicted stop that has not
// converged ends the predictions for the solve: from then on full batches.
// Only the launch schedule depends on it: the iterates and the stopping
// decision are the device's, and a short prediction only makes the host
// queue more.
class BatchPlanner {
 public:
  BatchPlanner(int full, double rtol) : full_(std::max(full, 1)), rtol2_(rtol * rtol) {}

  // iterations to queue from iteration k; 0: wait for the next record
  int next(int k) {
    if (missed_ || npoll_ < 2 || !(bb_ > 0.0) || !(rr1_ > 0.0) || !(rr0_ > 0.0) || k1_ <= k0_)
      return full_;
    const double slope = (std::log(rr1_) - std::log(rr0_)) / (double)(k1_ - k0_);
    const double target = rtol2_ * bb_;
    if (!(slope < 0.0) || !std::isfinite(slope) || !(target > 0.0)) return full_;
    if (rr1_ <= target) return restart();
    const double ahead = (std::log(target) - std::log(rr1_)) / slope;  // > 0
    if (!(ahead < 1e6)) return full_;
    // none close by: the record arrives while the batch's last G step
    // still runs, and the host then queues more
    const int kc = k1_ + (int)std::ceil(ahead - 1e-6);
    const int margin = (int)std::ceil(0.05 * ahead - 1e-6);
    const int need = kc + margin - k + 1;
    if (need < full_) pred_ = std::max(pred_, kc + margin);
    return std::max(0, std::min(need, full_));
  }

  // batch when nothing is queued and next() is 0
  int restart() const { return std::min(full_, 2); }

  // a record: iteration k not converged, ||r_k||^2 = rr, ||b||^2 = bb
  void observe(int k, double rr, double bb) {
    if (npoll_ > 0 && k <= k1_) return;
    if (pred_ > 0 && k >= pred_) missed_ = true;
    k0_ = k1_;
    rr0_ = rr1_;
    k1_ = k;
    rr1_ = rr;
    bb_ = bb;
    ++npoll_;
  }

 private:
  int full_;
  double rtol2_;
  int npoll_ = 0;
  int k0_ = 0, k1_ = 0;
  double rr0_ = 0.0, rr1_ = 0.0, bb_ = 0.0;
  int pred_ = 0;         // latest iteration a shortened batch was sized to reach
  bool missed_ = false;  // a record past that iteration had not converged
};

}  // namespace sla
