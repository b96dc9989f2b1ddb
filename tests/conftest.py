import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the error of every full-size workload comparison (and a count of
    the others), so the figures survive in a quiet (-q) run's output."""
    mod = sys.modules.get("gpu_helpers")
    log = getattr(mod, "PARITY_LOG", None) if mod else None
    if not log:
        return
    tr = terminalreporter
    tr.write_line(f"parity: {len(log)} comparisons against the oracle; full-size workloads:")
    for what, rows, mx, mean in log:
        if what.startswith(("fp32_B", "bf16_B")):
            tr.write_line(f"  {what}: rows={rows} max_abs={mx:.3e} mean_abs={mean:.3e}")
    worst = max(log, key=lambda t: t[2])
    tr.write_line(f"  largest max_abs of all comparisons: {worst[2]:.3e} ({worst[0]})")
