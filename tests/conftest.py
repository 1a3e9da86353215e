import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle():
    """The CPU oracle; MOEDX_ORACLE_LIB names another build of it (the
    sanitizer run of test_oracle_sanitized.py)."""
    from oracle import Oracle
    path = os.environ.get("MOEDX_ORACLE_LIB")
    return Oracle(path) if path else Oracle()
