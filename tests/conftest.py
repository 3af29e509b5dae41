import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU cases")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


def pytest_runtest_logstart(nodeid, location):
    # name the case on the raw stream before it runs, so a run that dies
    # inside a GPU call still says which case it was in
    sys.__stderr__.write(f"[case] {nodeid}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device (run them with -m gpu on an MI355X)")
    from cross_layer_index_amd import ic
    return ic


def pytest_terminal_summary(terminalreporter):
    from checks import ERRORS
    if ERRORS:
        terminalreporter.section("achieved errors (max-abs unless noted; bar 5e-3)")
        for what, err in ERRORS:
            terminalreporter.write_line(f"[max-abs] {what}: {err:.3e}")
