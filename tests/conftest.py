import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_terminal_summary(terminalreporter):
    """Near-T accounting of the commit parity tests: rows whose oracle confidence lies within 1e-4
    of T are not graded bit-exactly, and groups decided by such rows (or by a fallback between
    confidences within a relative 1e-4 of each other) are checked for validity only; their counts are
    reported here so that they survive a quiet run."""
    gu = sys.modules.get("gpu_util")
    log = getattr(gu, "NEAR_T_LOG", None) if gu is not None else None
    if not log:
        return
    per = {}
    for test, rows, near, amb in log:
        t = per.setdefault(test.split("::")[0], [0, 0, 0, 0])
        t[0] += 1
        t[1] += rows
        t[2] += near
        t[3] += amb
    tot = [sum(v[i] for v in per.values()) for i in range(4)]
    terminalreporter.write_sep("-", "commit near-T accounting (band 1e-4)")
    for name, (steps, rows, near, amb) in sorted(per.items()):
        terminalreporter.write_line(f"{name}: {steps} commit steps, {rows} masked rows graded, "
                                    f"{near} near-T rows, {amb} groups checked for validity only")
    terminalreporter.write_line(f"near-T total: {tot[0]} commit steps, {tot[1]} masked rows graded, "
                                f"{tot[2]} near-T rows, {tot[3]} validity-only groups")
