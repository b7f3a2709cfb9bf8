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
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: exhaustive sweep, opt-in with NVFP4_SLOW=1")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("NVFP4_SLOW") == "1":
        return
    skip = pytest.mark.skip(reason="exhaustive sweep; set NVFP4_SLOW=1 to run")
    for it in items:
        if "slow" in it.keywords:
            it.add_marker(skip)


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.build(force=False)
    return oracle


@pytest.fixture(scope="session")
def gpu():
    """The product binding on cuda:0; GPU tests fail loudly if the library is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import microscaling_fp4_block_amd as m

    m.load()  # raises if libnvfp4.so was not built
    return m
