"""Shared pytest setup: repository root on sys.path, the ``gpu`` marker,
and building the CPU oracle / HIP library when they are missing."""
from __future__ import annotations

import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an AMD Instinct MI355X (gfx950) GPU")
    import oracle
    if not oracle.LIB_PATH.exists():
        from oracle import build as obuild
        obuild.build()


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()
