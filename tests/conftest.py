import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """List the parity cases that passed through the oracle-spread reading
    (gates re-taken against the oracle's own one-ulp spread), if any ran."""
    mod = sys.modules.get("gpu_util")
    cases = getattr(mod, "FALLBACKS", None) if mod else None
    if not cases:
        return
    terminalreporter.write_line(f"oracle-spread fallback taken by {len(cases)} case(s):")
    for c in cases:
        terminalreporter.write_line(f"  {c}")
