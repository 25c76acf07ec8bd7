import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")
    config.addinivalue_line("markers", "fullsize(job): compares with a full-size oracle reference "
                                       "computed by the background oracle process")


def _gpu_present() -> bool:
    # counts devices without initialising the HIP runtime
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        return False


@pytest.hookimpl(trylast=True)       # after -m / -k deselection
def pytest_collection_modifyitems(config, items):
    has_gpu = _gpu_present()
    if has_gpu:
        # Full-size oracle references: one child process computes them while
        # the other GPU tests run (in collection order of the tests that use them).
        import _fullsize
        jobs = []
        for it in items:
            m = it.get_closest_marker("fullsize")
            if m and m.args[0] not in jobs:
                jobs.append(m.args[0])
        _fullsize.start(jobs)
        return
    # GPU tests cannot run without a device: skip them rather than fail when
    # they are collected on a CPU-only machine with an explicit -m gpu.
    skip = pytest.mark.skip(reason="no GPU on this machine")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_unconfigure(config):
    mod = sys.modules.get("_fullsize")
    if mod is not None:
        mod.stop()
