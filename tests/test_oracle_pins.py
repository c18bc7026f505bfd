"""The CPU oracle against mathematics independent of it (see pins.py)."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=[p.__name__ for p in pins.ALL_PINS])
def test_pin(pin):
    pin(oracle.load())


def test_oracle_bitwise_independent_of_thread_count():
    """Fixed-block dot products make the result identical for 1 and 4 threads."""
    code = (
        "import sys, numpy as np; sys.path.insert(0, %r); import oracle;"
        "from preconditioned_cg_solver_amd import inputs as I;"
        "p = I.make_problem(2, size=24); x, st, it, rr = oracle.pcg(p.A, p.G, p.eps, p.b, 1e-10, 5000);"
        "sys.stdout.write(x.tobytes().hex()[:20000] + ' %%d %%d' %% (st, it))"
    ) % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for t in ("1", "4"):
        env = dict(os.environ, OMP_NUM_THREADS=t)
        outs.append(subprocess.run([sys.executable, "-c", code], env=env, check=True,
                                   capture_output=True, text=True).stdout)
    assert outs[0] == outs[1]
