import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a GPU; fail loudly instead of skipping when
    # one was requested on purpose (-m gpu) but none is present.
    pass


@pytest.fixture(scope="session")
def has_gpu():
    import torch
    return torch.cuda.is_available()
