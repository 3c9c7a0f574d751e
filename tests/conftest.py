import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Near-tie argmax exemptions the GPU parity tests took (each one a row
    where the oracle's gap to the best other id was below the GPU's measured
    error on the two rows)."""
    mod = sys.modules.get("gpu_util")
    if mod is None:
        return
    ties = getattr(mod, "NEAR_TIES", [])
    terminalreporter.write_line(f"argmax near-tie exemptions taken: {len(ties)}")
    for what, t, gap, err in ties:
        terminalreporter.write_line(f"  {what} t={t}: gap {gap:.3g} < measured error {err:.3g}")
