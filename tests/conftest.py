import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library)")


def _parity_rows():
    try:
        from tests import gpu_helpers as H
    except Exception:
        return []
    return sorted(H.REPORT.items())


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Band-excluded coordinates, code flips inside the band and the largest errors of
    every GPU parity test and workload (when any ran)."""
    rows = _parity_rows()
    if not rows:
        return
    terminalreporter.write_line("parity figures (test, workload: values):")
    for (test, wl), rec in rows:
        terminalreporter.write_line(f"  {test}, {wl}: " + ", ".join(
            f"{k} {v:.2e}" if isinstance(v, float) else f"{k} {v}" for k, v in sorted(rec.items())))
    path = os.environ.get("TQ_PARITY_REPORT")
    if path:
        _write_report(path, rows)


def _write_report(path, rows):
    keys = sorted({k for _, rec in rows for k in rec})
    with open(path, "w") as f:
        f.write("# Parity report of the GPU tests\n\n")
        f.write("Written by `pytest -m gpu` (tests/conftest.py) when TQ_PARITY_REPORT names a file.\n")
        f.write("Counts add up over the test's cases; `worst_*` and `max_*` are maxima.\n")
        f.write("`*_band`: coordinates within 1e-6 of a decision boundary (excluded from the bit-exact\n")
        f.write("check); `*_band_flips`: of those, the ones whose code differs from the oracle's;\n")
        f.write("`worst_*_l2` / `worst_*_elem`: relative L2 and largest elementwise error (over the\n")
        f.write("largest reference magnitude) of a (sequence, q head) vector; `max_*_ulp`: stored fp32\n")
        f.write("norms against the oracle's fp32 rounding.\n\n")
        f.write("| test | workload | " + " | ".join(keys) + " |\n")
        f.write("|---|---|" + "---|" * len(keys) + "\n")
        for (test, wl), rec in rows:
            cells = []
            for k in keys:
                v = rec.get(k)
                cells.append("" if v is None else (f"{v:.2e}" if isinstance(v, float) else str(v)))
            f.write(f"| {test} | {wl} | " + " | ".join(cells) + " |\n")
