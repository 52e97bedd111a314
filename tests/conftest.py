import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built libkvarn.so")


@pytest.fixture(scope="session")
def oracle():
    import oracle as o
    o.build(force=False)
    return o


@pytest.fixture(scope="session")
def kvarn():
    """The product library (C-ABI through its Python binding). On a GPU machine a
    missing or stale library is an error, never a skip."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this container")
    import kv_cache_bit_kvarn_amd as kv
    kv.load()
    return kv
