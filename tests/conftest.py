"""Shared pytest setup: the ``gpu`` marker and the repository import path.

Tests marked ``gpu`` need an MI355X (gfx950) and the built HIP library. With
no GPU they are skipped, unless SATTN_REQUIRE_GPU=1 is set, in which case a
missing GPU is a failure (a skipped GPU run must never look like a pass).
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover - torch import problems
        return False


def pytest_collection_modifyitems(config, items):
    require = os.environ.get("SATTN_REQUIRE_GPU", "") == "1"
    if require or _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible (set SATTN_REQUIRE_GPU=1 to make this a failure)")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
