import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded for GPU tests.  Fails (not skips) if it is missing where a GPU is present."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import attention_flash_attn_prefill_amd as attn
    attn.load_library()  # raises if the shared library was not built
    return attn


@pytest.fixture
def progress(capsys):
    """A function that prints a progress line past pytest's output capture,
    for tests whose CPU-side oracle work runs for minutes."""
    def say(msg):
        with capsys.disabled():
            print(msg, flush=True)
    return say
