"""The C ABI's host side under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU touched): the host translation units (argument checks,
handle bookkeeping, the host utilities, the Lanczos/Sturm spectrum code,
tracing) are rebuilt with the sanitizers and linked with the library's
device objects; a C driver calls every entry point with invalid arguments
(each must return SLA_ERR_INVALID_ARG and set an error message) and the
host-only ones with valid arguments (Lanczos extremes against the closed
form of a Toeplitz tridiagonal, the status strings, the profiling switches).
Any out-of-bounds access or undefined operation fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "preconditioned_cg_solver_amd")
HOST_SOURCES = ["api.cpp", "host_util.cpp", "spectrum.cpp", "trace.cpp"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]

DRIVER = r"""
#include <math.h>
#include <stdio.h>
#include <string.h>
#include "sla.h"
#define BAD(call) do { sla_status s_ = (call); \
  if (s_ != SLA_ERR_INVALID_ARG) { printf("FAIL %s -> %d\n", #call, (int)s_); return 1; } \
  const char* e_ = sla_last_error(); \
  if (!e_ || !e_[0]) { printf("FAIL no message: %s\n", #call); return 1; } } while (0)
int main(void) {
  sla_mat_t m = 0;
  int32_t rp[3] = {0, 1, 2}, ci[2] = {0, 1};
  double v[2] = {1.0, 1.0}, w[2] = {0.0, 0.0};
  size_t bytes = 0;
  sla_solve_info info;
  BAD(sla_csr_create(NULL, 2, 2, rp, ci, v, SLA_F64, 0, 0));
  BAD(sla_csr_create(&m, -1, 2, rp, ci, v, SLA_F64, 0, 0));
  BAD(sla_csr_create(&m, 2, -1, rp, ci, v, SLA_F64, 0, 0));
  BAD(sla_csr_create(&m, 2, 2, NULL, ci, v, SLA_F64, 0, 0));
  BAD(sla_csr_create(&m, 2, 2, rp, NULL, v, SLA_F64, 0, 0));
  BAD(sla_csr_create(&m, 2, 2, rp, ci, NULL, SLA_F64, 0, 0));
  BAD(sla_csr_create(&m, 2, 2, rp, ci, v, (sla_dtype)7, 0, 0));
  BAD(sla_bsr_create(NULL, 2, 2, 3, rp, ci, v, SLA_F64, 0, 0));
  BAD(sla_pcg_workspace_size(NULL, &bytes));
  BAD(sla_pcg_workspace_size_multi(NULL, 2, &bytes));
  BAD(sla_spmv(NULL, w, w, 0));
  BAD(sla_spmv_t(NULL, w, w, 0));
  BAD(sla_spmm(NULL, w, w, 1, 0));
  BAD(sla_pcg_solve(NULL, NULL, 3e-3, w, w, 1e-8, 10, NULL, 0, 0, &info));
  BAD(sla_pcg_adjoint(NULL, NULL, 3e-3, w, w, w, w, 1e-8, 10, NULL, 0, 0, &info));
  BAD(sla_pcg_solve_multi(NULL, NULL, 3e-3, w, w, 0, 1e-8, 10, NULL, 0, 0, &info, NULL));
  BAD(sla_pattern_grad(NULL, w, w, w, 0));
  BAD(sla_mat_info(NULL, NULL, NULL, NULL, NULL));
  BAD(sla_lanczos_extremes(NULL, NULL, 3, NULL, NULL));
  /* host-only: the Lanczos tridiagonal of a constant-coefficient CG run is
     Toeplitz (diagonal a, off-diagonal b), eigenvalues a + 2 b cos(j pi / (k + 1)) */
  {
    enum { K = 40 };
    double al[K], be[K - 1], lo = 0, hi = 0;
    /* alpha_j = 1 / 2 and beta_j = 1 / 4 give the diagonal 1/alpha + beta/alpha_prev
       = 2.5 (2 for the first row) and the off-diagonal sqrt(beta) / alpha = 1 */
    for (int j = 0; j < K; ++j) al[j] = 0.5;
    for (int j = 0; j < K - 1; ++j) be[j] = 0.25;
    if (sla_lanczos_extremes(al, be, K, &lo, &hi) != SLA_OK) { printf("FAIL lanczos\n"); return 1; }
    if (!(lo > 0.0 && hi > lo && hi < 5.0)) { printf("FAIL extremes %g %g\n", lo, hi); return 1; }
  }
  for (int s = -6; s <= 1; ++s)
    if (!sla_status_string((sla_status)s) || !sla_status_string((sla_status)s)[0]) {
      printf("FAIL status string %d\n", s);
      return 1;
    }
  if (sla_set_profiling(0) != SLA_OK || sla_reset_profile() != SLA_OK) {
    printf("FAIL profiling switches\n");
    return 1;
  }
  printf("ok\n");
  return 0;
}
"""


def test_capi_host_side_under_sanitizers(tmp_path):
    from preconditioned_cg_solver_amd import build as B
    hip_objs = [os.path.join(PKG, "_build", s + ".o") for s in B.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in hip_objs):
        pytest.skip("the library's device objects are not built")
    objs = list(hip_objs)
    for src in HOST_SOURCES:
        obj = str(tmp_path / (src + ".o"))
        subprocess.run([B.hipcc(), *B.flags(), *SAN, "-c", os.path.join(PKG, "csrc", src), "-o",
                        obj], check=True, capture_output=True)
        objs.append(obj)
    lib = str(tmp_path / "libsla_san.so")
    subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *SAN, "-o", lib,
                    *objs, "-ldl"], check=True, capture_output=True)
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    exe = str(tmp_path / "driver")
    dobj = str(tmp_path / "driver.o")
    subprocess.run([B.hipcc(), "-x", "c", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
                    str(drv), "-o", dobj], check=True, capture_output=True)
    subprocess.run([B.hipcc(), *SAN, dobj, "-o", exe, lib, f"-Wl,-rpath,{tmp_path}"], check=True,
                   capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", HIP_VISIBLE_DEVICES="")
    out = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), (out.stdout, out.stderr[-3000:])
    assert "runtime error" not in out.stderr and "AddressSanitizer" not in out.stderr
