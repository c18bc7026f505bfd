"""Host-side unit test of the PCG driver's batch planner (plain C++ header,
compiled here with g++).  The planner only decides how many iterations the
host queues at a time; these checks pin its arithmetic on geometric
residual sequences, where the stopping iteration is known exactly."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "preconditioned_cg_solver_amd", "csrc")

DRIVER = r"""
#include <cmath>
#include <cstdio>
#include "planner.h"
using sla::BatchPlanner;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL line %d: %s\n", __LINE__, #c); return 1; } } while (0)
int main() {
  // no record yet, or one: full batches
  {
    BatchPlanner p(16, 1e-8);
    CHECK(p.next(1) == 16);
    CHECK(p.restart() == 2);
    p.observe(16, 1e-10, 1.0);
    CHECK(p.next(33) == 16);
  }
  // ||r_k||^2 = bb * 10^-k (a factor 10 per iteration), rtol 1e-4: the stop
  // test rr <= 1e-8 bb first holds at k = 8
  {
    BatchPlanner p(16, 1e-4);
    p.observe(2, 1e-2, 1.0);
    p.observe(4, 1e-4, 1.0);
    // from k = 5: iterations 5..8 reach the prediction, margin
    // ceil(0.05 * 4) = 1 -> 5 iterations
    CHECK(p.next(5) == 5);
    p.observe(6, 1e-6, 1.0);
    CHECK(p.next(10) == 0);             // 10 > 8 + margin 1: queued already
    CHECK(p.next(7) == 3);              // kc = 8, margin 1 -> 7..9
  }
  // the prediction lies inside what is already queued: wait
  {
    BatchPlanner p(8, 1e-4);
    p.observe(2, 1e-2, 1.0);
    p.observe(4, 1e-4, 1.0);
    CHECK(p.next(20) == 0);
  }
  // far from convergence: capped at the full batch
  {
    BatchPlanner p(8, 1e-12);
    p.observe(8, 0.5, 1.0);
    p.observe(16, 0.25, 1.0);
    CHECK(p.next(17) == 8);
  }
  // a record past a predicted stop that has not converged: full batches from
  // then on
  {
    BatchPlanner p(16, 1e-4);
    p.observe(2, 1e-2, 1.0);
    p.observe(4, 1e-4, 1.0);
    CHECK(p.next(5) == 5);              // sized to reach iteration 9
    p.observe(9, 1e-7, 1.0);            // not converged at 9
    CHECK(p.next(10) == 16);
    p.observe(12, 1e-8 * 1.0000001, 1.0);
    CHECK(p.next(13) == 16);
  }
  // no decrease, or garbage records: full batches (the device decides)
  {
    BatchPlanner p(8, 1e-8);
    p.observe(4, 1.0, 1.0);
    p.observe(8, 2.0, 1.0);
    CHECK(p.next(9) == 8);
    BatchPlanner q(8, 1e-8);
    q.observe(4, 0.5, 1.0);
    q.observe(8, std::nan(""), 1.0);
    CHECK(q.next(9) == 8);
    BatchPlanner z(8, 1e-8);
    z.observe(4, 0.5, 0.0);
    z.observe(8, 0.25, 0.0);
    CHECK(z.next(9) == 8);
  }
  // a stale record (iteration not past the last one) is ignored
  {
    BatchPlanner p(16, 1e-4);
    p.observe(2, 1e-2, 1.0);
    p.observe(4, 1e-4, 1.0);
    BatchPlanner q = p;
    q.observe(4, 1e-9, 1.0);
    CHECK(q.next(5) == p.next(5));
  }
  std::printf("ok\n");
  return 0;
}
"""


def test_batch_planner(tmp_path):
    src = tmp_path / "planner.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "planner"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC, str(src), "-o",
                    str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout
