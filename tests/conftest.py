import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device; skip them with a clear reason
    # instead of failing when they are selected on a CPU-only machine.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    # the parity figures of every GPU test that ran (relative error per slice,
    # per-row error, elementwise allclose violations), whatever the verbosity
    parity = sys.modules.get("parity")
    lines = getattr(parity, "REPORTS", []) if parity else []
    if lines:
        terminalreporter.section("parity figures")
        for line in lines:
            terminalreporter.write_line(line)
