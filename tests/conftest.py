import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (minutes of host-side input generation)")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a device; on a CPU-only host they are skipped, not failed.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


@pytest.fixture(autouse=True)
def _no_device_wait_timeouts(request):
    """Every workspace a GPU test creates is checked after the test: no bounded
    in-kernel wait may have given up (the library's sticky device error word,
    read through jssa_workspace_status)."""
    if "gpu" not in request.keywords:
        yield
        return
    import torch
    if not torch.cuda.is_available():
        yield
        return
    import token_level_sparse_dim_amd as J
    made = []
    orig = J.workspace

    def tracking(*args, **kwargs):
        ws = orig(*args, **kwargs)
        made.append(ws)
        return ws

    J.workspace = tracking
    try:
        yield
    finally:
        J.workspace = orig
    torch.cuda.synchronize()
    timeouts = [int(J.workspace_status(ws).cpu()[J.STATUS_WAIT_TIMEOUT]) for ws in made]
    made.clear()
    assert not any(timeouts), f"a bounded device wait gave up in {request.node.nodeid}: {timeouts}"
