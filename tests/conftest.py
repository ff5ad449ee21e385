"""Shared pytest configuration: the ``gpu`` marker and repository import path."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def vq():
    """The HIP library binding; GPU tests fail loudly if it cannot be loaded."""
    if not gpu_available():
        pytest.fail("GPU test collected on a machine without a GPU (run with -m 'not gpu')")
    from speculative_decoding_verify_vq_amd import vq as _vq
    return _vq
