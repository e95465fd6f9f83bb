import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)

_POOL = None


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    # CPU workers for whole-tensor oracle references, forked now, before any test can
    # initialise the GPU, and only when GPU tests are selected
    global _POOL
    expr = (config.getoption("markexpr", "") or "").replace(" ", "")
    if expr in ("", "gpu"):
        import oracle_pool
        _POOL = oracle_pool.make_pool()


def pytest_unconfigure(config):
    global _POOL
    if _POOL is not None:
        _POOL.terminate()
        _POOL.join()
        _POOL = None


@pytest.fixture(scope="session")
def oracle_pool():
    """The worker pool (None when there is no pool: references are then computed in
    this process)."""
    return _POOL


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    return torch.device("cuda:0")
