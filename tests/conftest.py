"""Shared pytest set-up.

Markers:
  gpu  -- needs an MI355X (gfx950) and the built HIP library; everything else
          runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The GPU library, initialised on cuda:0.  Fails loudly (never falls back)
    when the HIP library is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("gpu test collected on a machine without a GPU")
    import moe_decode_skinny_amd as sk

    sk.init(0)
    return sk
