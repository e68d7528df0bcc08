import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library binding (fails loudly if it cannot be loaded)."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("a gpu-marked test ran without a visible GPU")
    from linearized_attention_amd import api
    api.load()
    return api


SHIFT_AUTO = -1000000  # the library's "estimate the split shift" value of fwd_split_shift


@pytest.fixture
def lz_opts(gpu_lib):
    """Sets library options (lizard_set_option) for one test and restores their values after it."""
    names = ("fwd_kernel", "fwd_segments", "fwd_split_shift", "debug_sync")
    saved = {n: gpu_lib.get_option(n) for n in names}

    def set_opt(name, value):
        gpu_lib.set_option(name, value)

    yield set_opt
    for n, v in saved.items():
        gpu_lib.set_option(n, v)
