"""Host-side unit test of the int32 overflow guard of the sliced (SELL)
layouts: the guard header is plain C++ and is compiled here with g++."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "preconditioned_cg_solver_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include "bounds.h"
using sla::sliced_layout_fits;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL %s\n", #c); return 1; } } while (0)
int main() {
  const long long M = 2147483647LL;
  // 3D Poisson 128^3 in SELL-64: 32768 slices of at most 7 slots of 64 rows
  CHECK(sliced_layout_fits(32768, 7, 64, 1024));
  // 2^31 - 1 rows of width 32: far beyond int32
  CHECK(!sliced_layout_fits((M + 63) / 64, 32, 64, 1024));
  // the guard's boundary: total + tail = INT32_MAX - 1 fits, = INT32_MAX does not
  CHECK(sliced_layout_fits(1, 1, M - 1 - 1024, 1024));
  CHECK(!sliced_layout_fits(1, 1, M - 1024, 1024));
  CHECK(sliced_layout_fits((M - 1 - 1024) / 2048, 32, 64, 1024));
  CHECK(!sliced_layout_fits((M - 1 - 1024) / 2048 + 1, 32, 64, 1024));
  // products that would overflow 64-bit arithmetic are rejected, not wrapped
  CHECK(!sliced_layout_fits(1LL << 40, 1LL << 40, 64, 0));
  // empty layouts fit; negative sizes do not
  CHECK(sliced_layout_fits(0, 32, 64, 1024));
  CHECK(sliced_layout_fits(100, 0, 64, 1024));
  CHECK(!sliced_layout_fits(-1, 4, 64, 0));
  // BSR sliced ELL: 192 values per slot, 16 tail slots
  CHECK(sliced_layout_fits(12483, 27, 192, 16 * 192));
  CHECK(!sliced_layout_fits(1 << 20, 64, 192, 16 * 192));
  std::printf("ok\n");
  return 0;
}
"""


def test_sliced_layout_guard(tmp_path):
    src = tmp_path / "guard.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "guard"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC, str(src), "-o",
                    str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout
