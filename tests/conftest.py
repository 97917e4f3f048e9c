import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP path through the C ABI")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding, on a machine with a GPU.  A GPU test that reaches this
    fixture without a GPU or without the built library fails loudly."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import scaled_dot_product_attn_amd as attn
    attn.load_library()
    return attn
