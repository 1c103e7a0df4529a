import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (minutes on the CPU side)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library binding; skips only when no GPU is visible (never falls back)."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from qlora_fine_tuning_amd import lora

    lora.load()  # raises if the library was not built
    return lora
