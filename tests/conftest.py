"""Shared pytest configuration.

Markers:
  gpu -- needs an AMD GPU (gfx950) and the built HIP library; every other
         test runs on the CPU only.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
for _p in (ROOT, TESTS):
    if _p not in sys.path:
        sys.path.insert(0, _p)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs a gfx950 GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests run in the order they are written inside a file, files in
    # name order; nothing to reorder here.
    return


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
