import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path through the C-ABI")


MASK_TO_ORACLE = {"none": 0, "causal_tl": 1, "causal_br": 2}


def to_f64(t):
    """torch tensor (any float dtype, any device) -> numpy float64, exactly."""
    import torch
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


@pytest.fixture(scope="session")
def lib_path():
    """Path of the built C-ABI library; builds it if nothing is built yet."""
    from scaled_dot_product_02_amd import _binding
    path = _binding.library_path()
    if not os.path.exists(path):
        import __graft_entry__
        __graft_entry__.build()
    return path
