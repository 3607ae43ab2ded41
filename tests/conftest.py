import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _ensure_built():
    """Load what is built; build the two host-only C libraries only when absent."""
    import oracle
    import synth
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build()
    if not os.path.exists(os.path.join(ROOT, "synth", "libsynth.so")):
        synth.build()


_ensure_built()


@pytest.fixture(scope="session")
def torch_cpu():
    import torch
    return torch
