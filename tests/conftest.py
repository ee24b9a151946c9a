"""Shared pytest setup: the `gpu` marker and the repository root on sys.path."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library)")


def _gpu_present() -> bool:
    try:
        import torch
        return bool(torch.cuda.is_available()) and torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_present():
        return
    skip = pytest.mark.skip(reason="no GPU in this process")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_sessionfinish(session, exitstatus):
    out = os.environ.get("HLA2_PARITY_DIR")
    if out:
        from tests import parity
        parity.write_records(out)
