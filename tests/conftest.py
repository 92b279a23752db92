"""Shared test set-up: the `gpu` marker, the oracle build, and the HIP library handle."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: exhaustive CPU sweeps (seconds to a minute)")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    import oracle

    oracle.lib()  # builds with gcc if the shared object is missing
    yield


@pytest.fixture(scope="session")
def heal():
    """The product binding; fails loudly (no fallback) when the HIP library is missing."""
    import error_compensated_gemm_amd as heal_mod

    heal_mod.load()
    return heal_mod
