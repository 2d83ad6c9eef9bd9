"""Shared test configuration.

Tests marked ``gpu`` need an MI355X and the built HIP library; everything else
runs on any host (the CPU oracle, the host-side dispatcher, the C ABI's
argument validation and symbol table).
"""
from __future__ import annotations

import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size oracle comparisons")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle


@pytest.fixture(scope="session")
def device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")
