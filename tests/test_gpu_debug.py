"""The bounds-checking build (libsla_debug.so, loaded with SLA_DEBUG=1):
every gathered column index is checked on the device against the vector
length.  Valid input solves as the release build does; with
SLA_DEBUG_SHRINK=1 the check also rejects the last column (valid input, so
no access leaves the vector), which must surface as SLA_ERR_INVALID_ARG.
The library is chosen when the binding first loads it, so each case runs in
a child process."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

from preconditioned_cg_solver_amd import binding as B
from gpu_util import create, host, problem, rel, tdev

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import json, os, sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
import numpy as np
from preconditioned_cg_solver_amd import binding as B
from gpu_util import create, host, problem, tdev
assert B.lib_path().endswith("libsla_debug.so")
p = problem({key!r})
A, G = create(p.A), create(p.G, transpose=True)
out = {{}}
x, info = B.sla_pcg_solve(A, G, p.eps, tdev(p.b), rtol=p.rtol, maxit=p.maxit)
np.save({xfile!r}, host(x))
out["iterations"] = info.iterations
os.environ["SLA_DEBUG_SHRINK"] = "1"
x2, info2 = B.sla_pcg_solve(A, G, p.eps, tdev(p.b), rtol=p.rtol, maxit=p.maxit,
                            raise_on_error=False)
out["forced_status"] = info2.status
out["forced_error"] = B.sla_last_error()
print("RESULT " + json.dumps(out))
"""


@pytest.mark.skipif(not os.path.exists(os.path.join(ROOT, "preconditioned_cg_solver_amd",
                                                    "libsla_debug.so")),
                    reason="libsla_debug.so not built")
@pytest.mark.parametrize("key,order", [("poisson3d_13", "0"), ("powerlaw_20k", "1")])
def test_debug_build_checks_gathered_columns(key, order, tmp_path, monkeypatch):
    monkeypatch.setenv("SLA_ORDER", order)
    p = problem(key)
    A, G = create(p.A), create(p.G, transpose=True)
    x, info = B.sla_pcg_solve(A, G, p.eps, tdev(p.b), rtol=p.rtol, maxit=p.maxit)
    xfile = str(tmp_path / "x.npy")
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), key=key, xfile=xfile)
    env = dict(os.environ, SLA_DEBUG="1", SLA_ORDER=order)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    res = json.loads(r.stdout.split("RESULT ", 1)[1])
    # valid input: the release build's solve
    assert res["iterations"] == info.iterations
    assert rel(np.load(xfile), host(x)) <= 1e-12
    # the forced check: an error status, not a fault
    assert res["forced_status"] == B.ERR_INVALID_ARG
    assert "out of range" in res["forced_error"]
