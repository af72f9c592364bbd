"""Shared pytest configuration.

Markers:
  gpu - needs an MI355X (gfx950) and the built HIP library; everything else
        runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built libfp8bs.so")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; the test fails loudly if it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test selected but no GPU is visible")
    import fine_grained_fp8_amd as fp8
    fp8.load_library()  # raises if libfp8bs.so is not built
    return fp8
