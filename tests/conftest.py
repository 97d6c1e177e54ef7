import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def pytest_sessionfinish(session, exitstatus):
    # the GPU parity checks gather their figures in tests.parity.RECORD
    parity = sys.modules.get("tests.parity")
    if parity is not None:
        parity.write_record()
