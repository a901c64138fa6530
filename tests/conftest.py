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


def pytest_terminal_summary(terminalreporter):
    """Max errors of the full-size parity checks (whole (batch, head) slices of
    the workloads) and the worst case of every other check, in the session
    summary so they appear in quiet runs too."""
    try:
        from gpu_common import PARITY_LOG
    except Exception:
        return
    if not PARITY_LOG:
        return
    tr = terminalreporter
    tr.section("parity max errors (GPU vs CPU oracle)")
    full = {}
    for what, eo, el in PARITY_LOG:
        if "full slice" in what:
            name = what.split(" full slice")[0]
            n, o, l = full.get(name, (0, 0.0, 0.0))
            full[name] = (n + 1, max(o, eo), max(l, el or 0.0))
    for name, (n, o, l) in full.items():
        tr.write_line(f"{name}: {n} full (batch, head) slices, out max-abs {o:.3e}, lse max-abs {l:.3e}")
    worst_o = max(PARITY_LOG, key=lambda r: r[1])
    with_l = [r for r in PARITY_LOG if r[2] is not None]
    tr.write_line(f"{len(PARITY_LOG)} checks; worst out {worst_o[1]:.3e} ({worst_o[0]})")
    if with_l:
        worst_l = max(with_l, key=lambda r: r[2])
        tr.write_line(f"worst lse {worst_l[2]:.3e} ({worst_l[0]})")
