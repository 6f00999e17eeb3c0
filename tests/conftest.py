import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def htl():
    """The HIP library's Python binding; GPU tests skip only where no GPU exists."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")
    import hash_table_lookup_amd as h
    h.lib()            # a missing library is an error on a GPU host, not a skip
    return h


def to_np(t):
    """Device tensor -> numpy (bf16 as its uint16 bit pattern)."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
