"""Shared test setup: repo root on sys.path, the `gpu` marker, built libraries."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle


@pytest.fixture(scope="session")
def lib():
    """The C-ABI library (built from source if it is not there yet)."""
    from sharded_fsdp_flatten_amd import binding
    return binding


def golden_path(name):
    return os.path.join(GOLDEN, name)
