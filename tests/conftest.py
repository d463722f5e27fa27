import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the error statistics of every labelled parity comparison (the five
    configurations at both thresholds and both O types) at the end of the run,
    so the record of a GPU test session carries them."""
    parity = sys.modules.get("tests.parity")
    records = getattr(parity, "RECORDS", None) if parity else None
    if not records:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity vs the fp64 oracle (O max-abs bar 1e-2, mean 1e-3; LSE 1e-3*max(1,|LSE|))")
    tr.write_line(f"{'comparison':44s} {'elements':>11s} {'O max-abs':>10s} {'O mean-abs':>10s} "
                  f"{'>1e-2':>6s} {'allow':>6s} {'LSE rel':>9s} {'LSE fl-rel':>10s}")
    for label, st in records:
        tr.write_line(f"{label:44s} {st.get('n_elem', 0):11d} {st.get('o_max_abs', 0.0):10.3e} "
                      f"{st.get('o_mean_abs', 0.0):10.3e} {st.get('n_over_1e2', 0):6d} "
                      f"{st.get('n_allowance', 0):6d} {st.get('lse_max_rel', float('nan')):9.2e} "
                      f"{st.get('lse_max_floor_rel', float('nan')):10.2e}")
