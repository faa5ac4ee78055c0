"""Test configuration: the `gpu` marker and shared fixtures.

`-m "not gpu"` runs on any machine: the oracle against its pins, host logic,
and the C ABI's exports and argument checks (no kernel launches).
`-m gpu` runs the HIP path against the oracle and needs an MI355X.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a gfx950 GPU (runs the HIP kernels)")


@pytest.fixture(scope="session")
def rattn_lib():
    """The built librattn.so (built here if absent)."""
    from ring_attention_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from ring_attention_amd import build
        build.build()
    return binding.load_library()


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")
