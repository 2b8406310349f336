import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu_required(request):
    """GPU tests fail (never skip) when no GPU is visible: the HIP path must run."""
    if request.node.get_closest_marker("gpu") is not None:
        import torch
        if not torch.cuda.is_available():
            pytest.fail("test marked gpu but no HIP device is visible")
        print(f"\n[gpu] {request.node.nodeid}", flush=True)
    yield


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """How many outputs of each floating-point check passed only through the
    binary32 cancellation floor (tests/tolerance.py)."""
    try:
        from tests.tolerance import FLOOR_LOG
    except Exception:
        return
    if not FLOOR_LOG:
        return
    tr = terminalreporter
    tr.write_sep("-", "outputs within the cancellation floor only")
    agg = {}
    for what, fmt, n, size in FLOOR_LOG:
        a = agg.setdefault((what.split(" ")[0], fmt), [0, 0, 0.0])
        a[0] += n
        a[1] += size
        a[2] = max(a[2], n / max(size, 1))
    for (what, fmt), (n, size, worst) in sorted(agg.items()):
        tr.write_line(f"{what:28s} {fmt:5s} {n:9d} of {size:10d} ({100 * n / max(size, 1):.3f}%; "
                      f"worst single check {100 * worst:.3f}%)")
