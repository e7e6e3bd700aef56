import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests run on a box with a GPU; on a CPU-only host they are skipped,
    # not silently passed, so `-m gpu` there reports what did not run.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_runtest_logreport(report):
    # Print a failure's traceback the moment it happens: if a later test takes
    # the process down, the end-of-session summary would never be written.
    if report.failed:
        sys.stderr.write(f"\n[failure] {report.nodeid} ({report.when})\n{report.longreprtext}\n")
        sys.stderr.flush()
