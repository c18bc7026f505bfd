"""SLA_TRACE=1: roctx ranges (recorded by rocprofv3 --marker-trace) and one
stderr line per solve.  The switch is read once per process, so the solve
runs in a child process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
from preconditioned_cg_solver_amd import binding as B
from gpu_util import create, problem, tdev
p = problem("poisson3d_13")
A, G = create(p.A), create(p.G, transpose=True)
x, info = B.sla_pcg_solve(A, G, p.eps, tdev(p.b), rtol=p.rtol, maxit=p.maxit)
B.sla_pcg_adjoint(A, G, p.eps, x, tdev(p.b), rtol=p.rtol, maxit=p.maxit)
print("iterations", info.iterations)
"""


@pytest.mark.parametrize("on", ["1", "0"])
def test_trace_lines(on):
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    env = dict(os.environ, SLA_TRACE=on)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    its = int(r.stdout.split("iterations")[1].split()[0])
    lines = [l for l in r.stderr.splitlines() if l.startswith("[sla] ")]
    if on == "0":
        assert lines == []
        return
    solve = [l for l in lines if l.startswith("[sla] sla_pcg_solve ")]
    assert len(solve) == 1 and f"iterations={its} " in solve[0] and "status=SLA_OK" in solve[0]
    assert any(l.startswith("[sla] sla_pcg_adjoint ") for l in lines)
    assert sum(l.startswith("[sla] sla_csr_create ") for l in lines) == 2
