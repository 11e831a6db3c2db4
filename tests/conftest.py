import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_runtest_setup(item):
    # GPU tests run with the binding's NaN canary on: every workspace, state
    # and output it allocates starts as NaN, so a slot read before it is
    # written shows up in the comparison with the oracle.
    if item.get_closest_marker("gpu") is not None:
        from exact_blockwise_long_amd import blockattn
        blockattn.set_poison(True)


def pytest_runtest_teardown(item):
    if item.get_closest_marker("gpu") is not None:
        from exact_blockwise_long_amd import blockattn
        blockattn.set_poison(False)
