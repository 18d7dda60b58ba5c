import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library bound to cuda:0; fails loudly when it cannot load."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test selected but no GPU is visible")
    import head_latent_attention_07_amd as mla
    mla.load()
    return mla


@pytest.fixture(scope="session", autouse=True)
def debug_word_after_session():
    """With MLA_LIBRARY naming the debug-checks build, the whole session's
    error word must be empty at its end (tests that plant invalid lengths,
    block entries or positions read and clear the word themselves)."""
    yield
    lib = os.environ.get("MLA_LIBRARY", "")
    if not lib.endswith("_debug.so"):
        return
    import head_latent_attention_07_amd as mla
    if mla._lib is None:      # the library was never loaded (no GPU test ran)
        return
    word = mla.debug_errors()
    print(f"\n[debug] error word after the session: {word:#x}", flush=True)
    assert word == 0, f"debug checks reported violations: {word:#x}"
