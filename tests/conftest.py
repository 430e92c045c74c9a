"""Shared pytest configuration.

Markers: ``gpu`` marks tests that need an MI355X (gfx950) device.  Tests without
the marker run on any CPU host.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def pytest_collection_modifyitems(config, items):
    """GPU tests are skipped, with a reason, when no GPU is visible.

    They are never skipped because the HIP library is missing: the binding raises
    on import in that case, and the test fails.
    """
    gpu_items = [it for it in items if "gpu" in it.keywords]
    if not gpu_items:
        return
    try:
        import torch

        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if not have_gpu:
        skip = pytest.mark.skip(reason="no GPU visible on this host")
        for it in gpu_items:
            it.add_marker(skip)


def golden_path(name: str) -> str:
    return os.path.join(ROOT, "tests", "golden", name)


def read_golden_rows(name: str):
    """Non-comment, non-empty lines of a golden fixture, split on whitespace."""
    rows = []
    with open(golden_path(name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows
