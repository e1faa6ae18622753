import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (minutes of CPU time for the oracle)")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(autouse=True)
def _workspaces_end_clear(request, monkeypatch):
    """Every workspace a GPU test allocates through the binding (its own or the one a forward call
    makes when none is passed) must end the test with its failure word clear: no bounded wait of a
    forward call expired unnoticed. A test that forces an expiry reads the word itself, which clears it."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    from calibration_free_channel_amd import _lib
    import calibration_free_channel_amd as cfm
    made = []
    orig = _lib.new_workspace

    def recording(nbytes, device):
        ws = orig(nbytes, device)
        made.append(ws)
        return ws

    monkeypatch.setattr(_lib, "new_workspace", recording)
    monkeypatch.setattr(cfm, "new_workspace", recording)
    yield
    bad = [n for n, ws in enumerate(made) if _lib.workspace_status(ws) != 0]
    made.clear()
    assert not bad, f"{len(bad)} of the test's workspaces report an expired bounded wait"
