import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size) case")


import pytest  # noqa: E402


@pytest.fixture
def launch_override():
    """Pins the block-step kernel and launch shape through bdssm_set_launch_override for
    one test; back to automatic afterwards."""
    from bidirectional_mamba_state_amd import bdssm
    yield bdssm.set_launch_override
    bdssm.set_launch_override()
