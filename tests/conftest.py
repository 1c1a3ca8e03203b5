import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

_CONFIG = None


def pytest_configure(config):
    global _CONFIG
    _CONFIG = config
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def say(msg: str) -> None:
    """One line on the process's real stderr, past pytest's output capture
    (which also redirects file descriptor 2), flushed at once."""
    capman = _CONFIG.pluginmanager.getplugin("capturemanager") if _CONFIG else None
    if capman is None:
        sys.stderr.write(msg + "\n")
        sys.stderr.flush()
        return
    with capman.global_and_fixture_disabled():
        sys.stderr.write(msg + "\n")
        sys.stderr.flush()


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device; skip them loudly instead of failing
    # in a CPU-only container (the GPU run selects them with -m gpu).
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    # Name the case on the real stderr before it touches the GPU, so a run that
    # dies inside a kernel still says which case it was.
    if "gpu" in request.keywords:
        say(f"[gpu case] {request.node.nodeid}")
    yield
