import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    """KDA_ORACLE_LIB_OVERRIDE swaps the oracle for a planted-mistake build; only the CPU
    mutation test may set it (for the pin suite it runs in a subprocess).  A session that
    would compare the GPU against a swapped oracle is refused."""
    if os.environ.get("KDA_ORACLE_LIB_OVERRIDE") and any(
            item.get_closest_marker("gpu") for item in items):
        raise pytest.UsageError("KDA_ORACLE_LIB_OVERRIDE is set: GPU parity tests would compare "
                                "against a swapped oracle; unset it")
