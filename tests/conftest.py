"""Shared pytest configuration: the ``gpu`` marker and repo-root imports."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: large oracle sample; runs in the GPU suite only")


def pytest_report_header(config):
    return f"repo root: {ROOT}"


@pytest.fixture(scope="session")
def repo_root():
    return ROOT


@pytest.fixture(scope="session")
def dfa_lib():
    """The C-ABI library, built in-tree only if no build exists yet."""
    from long_context_exact_amd import build as b
    if not os.path.exists(b.LIB_PATH):
        b.build()
    from long_context_exact_amd import dfa
    return dfa
