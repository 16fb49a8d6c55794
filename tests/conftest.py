import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Observed normwise errors of the GPU parity comparisons against their tolerances."""
    try:
        from tests import gpu_harness as G
    except Exception:
        return
    if not G.OBSERVED:
        return
    tr = terminalreporter
    tr.section("observed parity errors (normwise, against tolerance)")
    frac = lambda t: t[1] / t[2] if t[2] else 0.0  # noqa: E731
    line = lambda t: f"{t[1]:10.3e}  tol {t[2]:.0e}  {frac(t):6.3f}  {t[0]}"  # noqa: E731
    for t in G.OBSERVED:
        tr.write_line(line(t))
    tr.write_line(f"{len(G.OBSERVED)} comparisons; the closest to their tolerance:")
    for t in sorted(G.OBSERVED, key=frac, reverse=True)[:10]:
        tr.write_line(line(t))
