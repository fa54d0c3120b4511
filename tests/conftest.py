import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP libraries")
    config.addinivalue_line("markers", "slow: full-size parity cases")


@pytest.fixture(scope="session", autouse=True)
def _host_libraries_built():
    """The CPU-side libraries (generator and oracle) are cheap to build with
    gcc; build them if they are missing so the CPU suite runs on a fresh
    checkout.  HIP libraries are built by __graft_entry__.build()."""
    from oracle import LIB as ORACLE_LIB
    from synth import HOST_LIB

    if not os.path.exists(ORACLE_LIB):
        from oracle.build import build as build_oracle

        build_oracle()
    if not os.path.exists(HOST_LIB):
        from synth.build import build as build_synth

        build_synth(device=False)
    yield


def gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False
