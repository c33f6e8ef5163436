import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_addoption(parser):
    parser.addoption("--c3-reading", choices=["capped", "full", "both"], default="both",
                     help="reading of the 16K workload's budgets the parity tests run (default: both)")


def c3_readings(config):
    r = config.getoption("--c3-reading")
    return ["capped", "full"] if r == "both" else [r]


def pytest_generate_tests(metafunc):
    if "c3_reading" in metafunc.fixturenames:
        metafunc.parametrize("c3_reading", c3_readings(metafunc.config))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    # the GPU tests' progress lines bypass output capture (a long test then
    # never looks silent to a watchdog on its output)
    here = os.path.dirname(os.path.abspath(__file__))
    if here not in sys.path:
        sys.path.insert(0, here)
    import _parity
    _parity._capman = config.pluginmanager.getplugin("capturemanager")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a visible device; without one they are skipped, never
    # rerouted to a CPU path.
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
