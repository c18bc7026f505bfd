"""The C-ABI library loads and exports every entry point include/sla.h declares
(no compute calls: runs without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(sla_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def libsla():
    from preconditioned_cg_solver_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    import torch  # noqa: F401  (same runtime order as the binding)
    return ctypes.CDLL(build.LIB)


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("sla_csr_create", "sla_bsr_create", "sla_mat_destroy", "sla_spmv",
                     "sla_pcg_workspace_size", "sla_pcg_solve", "sla_pcg_adjoint",
                     "sla_status_string", "sla_last_error"):
        assert required in names


def test_every_declared_symbol_is_exported(libsla):
    missing = [n for n in declared_functions() if not hasattr(libsla, n)]
    assert not missing, missing


def test_status_strings_without_gpu(libsla):
    libsla.sla_status_string.restype = ctypes.c_char_p
    libsla.sla_status_string.argtypes = [ctypes.c_int]
    assert libsla.sla_status_string(0) == b"SLA_OK"
    assert libsla.sla_status_string(-3) == b"SLA_ERR_BREAKDOWN"


def test_null_handle_is_rejected_without_gpu(libsla):
    libsla.sla_pcg_workspace_size.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    libsla.sla_pcg_workspace_size.restype = ctypes.c_int
    assert libsla.sla_pcg_workspace_size(None, None) == -1
    libsla.sla_last_error.restype = ctypes.c_char_p
    assert libsla.sla_last_error()


def test_every_entry_point_has_a_binding_of_the_same_name():
    from preconditioned_cg_solver_amd import binding
    missing = [n for n in declared_functions() if not callable(getattr(binding, n, None))]
    assert not missing, missing


def test_binding_has_the_same_names():
    from preconditioned_cg_solver_amd import binding
    for name in ("sla_csr_create", "sla_bsr_create", "sla_spmv", "sla_pcg_workspace_size",
                 "sla_pcg_solve", "sla_pcg_adjoint", "sla_precond_apply", "sla_pattern_grad",
                 "sla_mat_tiling", "sla_mat_reordered", "sla_mat_transpose_arrays",
                 "sla_set_profiling",
                 "sla_get_profile", "sla_reset_profile", "sla_status_string"):
        assert callable(getattr(binding, name))


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "preconditioned_cg_solver_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
                assert "oracle.c" not in src and "liboracle" not in src, f
