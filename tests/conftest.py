import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(autouse=True)
def _gpu_guard(request):
    """GPU tests skip up front on a machine without a GPU (before drawing large inputs)."""
    if request.node.get_closest_marker("gpu") is not None:
        import torch
        if not torch.cuda.is_available():
            pytest.skip("no GPU")


@pytest.fixture
def tune():
    """Force launch shapes of the library for one test (``tune(attn_cb=2, attn_splits=3)``);
    the overrides are removed when the test ends."""
    from tree_attention_verification_spec_amd import binding
    names = []

    def force(**knobs):
        for k, v in knobs.items():
            binding.tune(k, v)
            names.append(k)
    yield force
    for k in names:
        binding.tune(k, None)
