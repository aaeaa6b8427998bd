import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_sessionstart(session):
    # A run without a GPU builds the HIP library (hipcc cross-compiles for gfx950) when nothing is
    # built yet; a run on a GPU expects it built beforehand and fails loudly without it.
    import torch

    import long_context_compressed_06_amd as csa

    if not os.path.exists(csa.LIB_PATH) and torch.cuda.device_count() == 0:
        from long_context_compressed_06_amd import build

        build.build()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload check")


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle._load()
    return oracle
