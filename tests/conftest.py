import os
import sys

import pytest

# Under pytest-xdist every worker would start one OpenMP thread per core in
# the oracle, and their spin-waits oversubscribe the host: one thread each.
if os.environ.get("PYTEST_XDIST_WORKER"):
    os.environ.setdefault("OMP_NUM_THREADS", "1")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle():
    from oracle import oracle as O
    return O.default()


def pytest_terminal_summary(terminalreporter):
    """The error figures of every GPU comparison of the session, per test:
    the largest scaled error (the gated one), plain relative error and
    normwise error over the test's comparisons."""
    try:
        import gpu_util
    except Exception:
        return
    if not gpu_util.ERRORS:
        return
    per = {}
    for test, e, rel, norm, n in gpu_util.ERRORS:
        a = per.setdefault(test, [0.0, 0.0, 0.0, 0, 0])
        a[0], a[1], a[2] = max(a[0], e), max(a[1], rel), max(a[2], norm)
        a[3] += 1
        a[4] += n
    tr = terminalreporter
    tr.write_sep("-", "GPU parity errors (max over each test's comparisons)")
    tr.write_line(f"{'scaled':>9} {'relative':>9} {'normwise':>9} {'cmp':>4} {'elements':>11}  test")
    for test, (e, rel, norm, c, n) in per.items():
        tr.write_line(f"{e:9.2e} {rel:9.2e} {norm:9.2e} {c:4d} {n:11d}  {test}")
