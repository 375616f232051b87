import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """The parity figures the GPU tests measured (captured output is not shown
    for passing tests): the full-size workloads one per line, the rest as the
    worst E_row and E_scale per test file."""
    import gpu_util

    recs = gpu_util.PARITY
    if not recs:
        return
    tr = terminalreporter
    tr.write_sep("-", f"parity against the fp64 oracle ({len(recs)} comparisons)")
    worst = {}
    for test, what, e_row, e_scale in recs:
        if any(k in what for k in ("whole", "workload", "full size")):
            tr.write_line(f"{what}: E_row={e_row:.3e} E_scale={e_scale:.3e}")
        f = test.split("::")[0].split("/")[-1]
        w = worst.setdefault(f, [0.0, 0.0, 0])
        w[0], w[1], w[2] = max(w[0], e_row), max(w[1], e_scale), w[2] + 1
    for f, (er, es, n) in sorted(worst.items()):
        tr.write_line(f"{f}: {n} comparisons, worst E_row={er:.3e} E_scale={es:.3e}")
