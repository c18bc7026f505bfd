"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks that
at least one pin catches each of them.  The shipped oracle is never modified."""
import os

import numpy as np
import pytest

import oracle
import pins

MUTATIONS = [
    ("spmv drops the block column offset",
     "s += blk[c] * x[J * bs + c];", "s += blk[c] * x[J * bs];"),
    ("spmv reads x at the row instead of the column",
     "s += blk[c] * x[J * bs + c];", "s += blk[c] * x[I * bs + c];"),
    ("transpose keeps blocks untransposed",
     "t_val[dst * bb + (int64_t)c * bs + r]", "t_val[dst * bb + (int64_t)r * bs + c]"),
    ("dot skips the last element of every block",
     "for (int64_t i = lo; i < hi; ++i) s += a[i] * b[i];",
     "for (int64_t i = lo; i + 1 < hi; ++i) s += a[i] * b[i];"),
    ("preconditioner subtracts the shift",
     "z[i] = z[i] + eps * r[i];", "z[i] = z[i] - eps * r[i];"),
    ("preconditioner applies G twice instead of G G^T",
     "orc_spmv(Gt->nbr, Gt->bs, Gt->row_ptr, Gt->col, Gt->val, r, t);",
     "orc_spmv(G->nbr, G->bs, G->row_ptr, G->col, G->val, r, t);"),
    ("residual update with the wrong sign",
     "r[i] = r[i] - alpha * q[i];", "r[i] = r[i] + alpha * q[i];"),
    ("beta inverted",
     "const double beta = rho_new / rho;", "const double beta = rho / rho_new;"),
    ("search direction from r instead of z",
     "p[i] = z[i] + beta * p[i];", "p[i] = r[i] + beta * p[i];"),
    ("absolute instead of relative stopping test",
     "if (rnorm <= rtol * bnorm)", "if (rnorm <= rtol)"),
    ("alpha from the wrong inner product",
     "const double alpha = rho / sigma;", "const double alpha = rho / orc_dot(n, q, q);"),
    ("iteration counted before the update",
     "*iters = k;", "*iters = k + 1;"),
    ("adjoint gradient drops the block row offset",
     "-(lam[I * bs + r] * x[J * bs + c])", "-(lam[I * bs] * x[J * bs + c])"),
    ("adjoint gradient transposed (lambda_j x_i)",
     "-(lam[I * bs + r] * x[J * bs + c])", "-(lam[J * bs + c] * x[I * bs + r])"),
    ("adjoint gradient sign dropped",
     "-(lam[I * bs + r] * x[J * bs + c])", "(lam[I * bs + r] * x[J * bs + c])"),
    ("adjoint solves with b instead of dL/dx",
     "eps, gx, lam,", "eps, x, lam,"),
    ("Lanczos diagonal divides by the current alpha",
     "diag[j] = diag[j] + beta[j - 1] / alpha[j - 1];",
     "diag[j] = diag[j] + beta[j - 1] / alpha[j];"),
    ("Lanczos off-diagonal without the square root",
     "off[j] = sqrt(beta[j]) / alpha[j];", "off[j] = beta[j] / alpha[j];"),
    ("history records alpha one step late",
     "if (k <= hist_len) hist_a[k - 1] = alpha;", "if (k < hist_len) hist_a[k] = alpha;"),
    ("SAI loss ignores the scale",
     "d[i] = y[i] / s - wj[i];", "d[i] = y[i] - wj[i];"),
    ("SAI loss multiplies M^-1 A instead of A M^-1",
     "orc_precond_apply(nbr, bs, g_row_ptr, g_col, g_val, eps, wj, z);\n"
     "        if (st != ORC_OK) goto out;\n"
     "        orc_spmv(nbr, bs, a_row_ptr, a_col, a_val, z, y);",
     "ORC_OK;\n"
     "        orc_spmv(nbr, bs, a_row_ptr, a_col, a_val, wj, z);\n"
     "        st = orc_precond_apply(nbr, bs, g_row_ptr, g_col, g_val, eps, z, y);\n"
     "        if (st != ORC_OK) goto out;"),
    ("multi-RHS reads b column-major",
     "for (int64_t i = 0; i < n; ++i) bj[i] = b[i * k + j];",
     "for (int64_t i = 0; i < n; ++i) bj[i] = b[j * n + i];"),
    ("multi-RHS writes every column to the first",
     "for (int64_t i = 0; i < n; ++i) x[i * k + j] = xj[i];",
     "for (int64_t i = 0; i < n; ++i) x[i * k] = xj[i];"),
    ("multi-RHS adjoint gradient keeps only the last solve",
     "g = g - lam[(I * bs + r) * k + j] * x[(J * bs + c) * k + j];",
     "g = -lam[(I * bs + r) * k + j] * x[(J * bs + c) * k + j];"),
    ("multi-RHS adjoint gradient pairs lambda and x of different solves",
     "g = g - lam[(I * bs + r) * k + j] * x[(J * bs + c) * k + j];",
     "g = g - lam[(I * bs + r) * k + j] * x[(J * bs + c) * k + (k - 1 - j)];"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    oracle.build(str(mutant), so)
    lib = oracle.load(so)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError as e:
            caught.append(pin.__name__)
        except Exception as e:  # a crash of the mutant is also a catch
            caught.append(f"{pin.__name__} ({type(e).__name__})")
    assert caught, f"no pin caught: {name}"


# Plausible mistakes in Kaporin's number (a numpy function of the oracle
# package, so the mutants are Python functions rather than copies of oracle.c).
KAPORIN_MUTANTS = [
    ("harmonic instead of geometric mean",
     lambda e: float(np.mean(e) * np.mean(1.0 / np.asarray(e)))),
    ("ratio inverted",
     lambda e: float(np.exp(np.mean(np.log(e))) / np.mean(e))),
    ("sum instead of mean in the numerator",
     lambda e: float(np.sum(e) / np.exp(np.mean(np.log(e))))),
    ("log of the geometric mean used without exp",
     lambda e: float(np.mean(e) / np.mean(np.log(e)))),
    ("extreme-eigenvalue ratio",
     lambda e: float(np.max(e) / np.min(e))),
    ("square root of the ratio",
     lambda e: float(np.sqrt(np.mean(e) / np.exp(np.mean(np.log(e)))))),
]


@pytest.mark.parametrize("name,fn", KAPORIN_MUTANTS, ids=[m[0] for m in KAPORIN_MUTANTS])
def test_kaporin_pin_catches_planted_mistake(name, fn):
    with pytest.raises(AssertionError):
        with np.errstate(all="ignore"):
            pins.pin_kaporin(oracle.load(), kaporin=fn)
