import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Print the name of every GPU case before it touches the device, with
    pytest's output capture suspended (its fd-level capture also takes
    sys.__stderr__), so a run that dies mid-test still names its case."""
    if request.node.get_closest_marker("gpu") is not None:
        capman = request.config.pluginmanager.getplugin("capturemanager")
        if capman is None:
            sys.stderr.write(f"\n[gpu case] {request.node.nodeid}\n")
            sys.stderr.flush()
        else:
            with capman.global_and_fixture_disabled():
                sys.stderr.write(f"\n[gpu case] {request.node.nodeid}\n")
                sys.stderr.flush()
    yield


def pytest_terminal_summary(terminalreporter):
    """The measured error of every GPU parity check of the run (collected by
    tests/gpu_helpers.check), after the results."""
    helpers = sys.modules.get("tests.gpu_helpers")
    lines = getattr(helpers, "CHECKS", None)
    if lines:
        terminalreporter.section("measured errors of the GPU parity checks")
        for line in lines:
            terminalreporter.write_line(line)
